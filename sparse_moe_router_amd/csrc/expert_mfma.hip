// Expert SwiGLU FFNs as grouped GEMMs on the matrix cores, for many tokens
// per expert (prefill).  Each expert's tokens form a dense problem
// X_e [n_e x K] . W_e^T, and with thousands of tokens per layer most experts
// get tens to thousands of them (the router's skew makes the sizes uneven), so
// the weights are reused across a tile of tokens and the work is a contraction
// (expert sub-networks: page 2 "Layer 1"; low-bit weights: page 1 "How Strata
// Makes the Impossible Possible").
//
// Exactness.  The dequantised weight s * q is not a bf16 number in general, so
// the MFMA consumes the codes themselves and the fp16 group scale is applied
// in fp32 after each K = 32 step, which is exactly one group.  A code u is
// OR-ed into the top mantissa bits of bf16 1.0, giving the exact bf16 value
// 1 + u / 16 (4-bit), 1 + u / 8 (3-bit) or 1 + u / 4 (2-bit); with bf16 x every
// product is exact in fp32, and the offset term enters through the MFMA's
// accumulator input:
//   4-bit:  D = sum (1 + u/16) x - 1.5 sum x = sum (u - 8) x / 16,  acc += 16 s D
//   3-bit:  D = sum (1 + u/8) x - 1.5 sum x  = sum (u - 4) x / 8,   acc += 8 s D
//   2-bit:  D = sum (1 + u/4) x - sum x      = sum u x / 4,         acc += 4 s D + m sum x
// Keeping the code in the top mantissa bits keeps the cancelled offset within
// a few times the signal, so the fp32 sums lose little to the cancellation.
// The offset term is formed by one more MFMA per (16-token tile, group), with
// B = -1.5 (or -1) in every element, in the accumulator layout.
//
// Pipeline.  The activations, codes, scales (and minima) of a chunk of 4
// groups reach LDS by the DMA path (global_load_lds), double buffered, each
// buffer its own variable, and the reads of the current buffer are issued
// from asm blocks that wait for themselves: the compiler cannot tell that
// they do not touch the buffer the next chunk's copies are filling, and would
// otherwise wait for those copies before every read, so that no copy would
// run under the products.
//
// v_mfma_f32_16x16x32_bf16 lane layout (gfx950): A lane l holds row l % 16,
// k = 8 (l / 16) .. + 7; B lane l holds column l % 16 at the same k; D lane l
// holds rows 4 (l / 16) + i, column l % 16.  The codes of one B lane are 8
// consecutive codes and are unpacked into the pairs (k_j, k_{j+4}); the
// activations, copied raw, are put in that same pair order when read.
#include "gemv_tile.h"
#include <type_traits>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;          // tokens per tile
constexpr int kXcdTiles = 4;     // tiles per XCD work group
constexpr int kChunkG = 4;       // groups (of 32 k) per staged chunk

__device__ __forceinline__ f32x4_t mfma16(const uint32_t (&a)[4], const uint32_t (&b)[4], f32x4_t c) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v av = {a[0], a[1], a[2], a[3]};
  const u32x4v bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                 c, 0, 0, 0);
}

// Reads of the buffers the DMA path fills, each batch issued and waited for
// in one asm block (outputs early-clobber, so no address register doubles as
// an earlier read's destination).  Read through the compiler, each read would
// first wait for every copy in flight, the next chunk's included, which are
// meant to run under this chunk's products.  Addresses are LDS byte offsets.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }
typedef uint32_t frag4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void lds_read4x2(const uint32_t (&a)[4], uint2 (&o)[4]) {
  u32x2v_t r0, r1, r2, r3;
  asm volatile(
      "ds_read_b64 %0, %4\n\tds_read_b64 %1, %5\n\tds_read_b64 %2, %6\n\tds_read_b64 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
  o[0] = make_uint2(r0[0], r0[1]); o[1] = make_uint2(r1[0], r1[1]);
  o[2] = make_uint2(r2[0], r2[1]); o[3] = make_uint2(r3[0], r3[1]);
}
// four activation fragments (16 B at abase + AO + 4096 mt, mt = 0..3) and NB
// code dwords (at cb[i] + BO for the first four, cb[i] + BO2 for the rest);
// the offsets are the instructions' immediates, so one base register serves
// every group of a chunk
template <int NB, int AO, int BO, int BO2>
__device__ __forceinline__ void grp_read(uint32_t abase, const uint32_t (&cb)[NB], frag4_t (&f)[4],
                                         uint32_t (&c)[NB]) {
  if constexpr (NB == 4) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%13\n\tds_read_b128 %1, %8 offset:%14\n\t"
        "ds_read_b128 %2, %8 offset:%15\n\tds_read_b128 %3, %8 offset:%16\n\t"
        "ds_read_b32 %4, %9 offset:%17\n\tds_read_b32 %5, %10 offset:%17\n\t"
        "ds_read_b32 %6, %11 offset:%17\n\tds_read_b32 %7, %12 offset:%17\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3])
        : "v"(abase), "v"(cb[0]), "v"(cb[1]), "v"(cb[2]), "v"(cb[3]), "i"(AO), "i"(AO + 4096), "i"(AO + 8192),
          "i"(AO + 12288), "i"(BO)
        : "memory");
  } else {
    static_assert(NB == 8, "4 or 8 code dwords");
    asm volatile(
        "ds_read_b128 %0, %12 offset:%21\n\tds_read_b128 %1, %12 offset:%22\n\t"
        "ds_read_b128 %2, %12 offset:%23\n\tds_read_b128 %3, %12 offset:%24\n\t"
        "ds_read_b32 %4, %13 offset:%25\n\tds_read_b32 %5, %14 offset:%25\n\t"
        "ds_read_b32 %6, %15 offset:%25\n\tds_read_b32 %7, %16 offset:%25\n\t"
        "ds_read_b32 %8, %17 offset:%26\n\tds_read_b32 %9, %18 offset:%26\n\t"
        "ds_read_b32 %10, %19 offset:%26\n\tds_read_b32 %11, %20 offset:%26\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]),
          "=&v"(c[4]), "=&v"(c[5]), "=&v"(c[6]), "=&v"(c[7])
        : "v"(abase), "v"(cb[0]), "v"(cb[1]), "v"(cb[2]), "v"(cb[3]), "v"(cb[4]), "v"(cb[5]), "v"(cb[6]),
          "v"(cb[7]), "i"(AO), "i"(AO + 4096), "i"(AO + 8192), "i"(AO + 12288), "i"(BO), "i"(BO2)
        : "memory");
  }
}

// 8 codes of one B lane -> 4 bf16 pairs (k_j, k_{j+4}): 1 + u/16 (4-bit),
// 1 + u/8 (3-bit: w holds the 8 low-bit fields in bits 0..15 and the 8 third
// bits in bits 16..23) or 1 + u/4 (2-bit).
template <int QF>
__device__ __forceinline__ void unpack_b(uint32_t w, uint32_t (&b)[4]) {
  // (no empty asm statement here to pin the unpack: with one, a build whose
  // group reads used immediate offsets gave wrong values in one accumulator
  // of the 4-bit gate/up full tiles, and its code had that empty statement
  // among the few instructions between an MFMA and the first VALU read of its
  // result; an empty statement emits nothing but may count as a wait state)
  if constexpr (QF == MOE_Q4_SYM_G32) {  // nibble j -> bits 3..6, nibble j + 4 -> bits 19..22
    b[0] = and_or(w << 3, 0x00780078u, 0x3f803f80u);
    b[1] = and_or(w >> 1, 0x00780078u, 0x3f803f80u);
    b[2] = and_or(w >> 5, 0x00780078u, 0x3f803f80u);
    b[3] = and_or(w >> 9, 0x00780078u, 0x3f803f80u);
  } else if constexpr (QF == MOE_Q3_SYM_G32) {
    // low fields 0..3 -> bits 0..7, 4..7 -> bits 16..23; third bits 0..3 ->
    // bits 0..3, 4..7 -> bits 16..19; field j -> bits 4..5, third bit j -> bit 6
    const uint32_t s = (w & 0xffu) | ((w & 0xff00u) << 8);
    const uint32_t h = ((w >> 16) & 0xfu) | ((w >> 4) & 0xf0000u);
    b[0] = and_or(h << 6, 0x00400040u, and_or(s << 4, 0x00300030u, 0x3f803f80u));
    b[1] = and_or(h << 5, 0x00400040u, and_or(s << 2, 0x00300030u, 0x3f803f80u));
    b[2] = and_or(h << 4, 0x00400040u, and_or(s, 0x00300030u, 0x3f803f80u));
    b[3] = and_or(h << 3, 0x00400040u, and_or(s >> 2, 0x00300030u, 0x3f803f80u));
  } else {  // 16 bits = 8 crumbs; the second byte moves to bits 16..23, crumb j -> bits 5..6
    const uint32_t s = (w & 0xffu) | ((w & 0xff00u) << 8);
    b[0] = and_or(s << 5, 0x00600060u, 0x3f803f80u);
    b[1] = and_or(s << 3, 0x00600060u, 0x3f803f80u);
    b[2] = and_or(s << 1, 0x00600060u, 0x3f803f80u);
    b[3] = and_or(s >> 1, 0x00600060u, 0x3f803f80u);
  }
}

// Work tiles: ceil(n_e / 64) per routed expert with n_e >= mfma_min tokens,
// in expert order, then ceil(T / 64) for the shared expert (if T >= mfma_min).  Every wave of a block derives its tile
// from the expert offsets (a wave-wide scan of the per-expert tile counts), so
// the tiling needs no list in memory.  Returns false past the last tile.
__device__ __forceinline__ bool find_tile(const FfnArgs& a, bool with_shared, int t, int& expert, int& m0) {
  constexpr int kPer = 16;  // experts per lane per pass (one pass up to E = 1024)
  const int lane = threadIdx.x & 63;
  const int per = (a.E + 63) / 64;
  const int e0 = lane * per, e_end = min(e0 + per, a.E);
  // offsets of this lane's experts, all requested at once; indices past the
  // lane's range repeat its last offset (no tiles)
  auto counts = [&](int base, int (&c)[kPer]) {
    int v[kPer + 1];
#pragma unroll
    for (int i = 0; i <= kPer; ++i) v[i] = a.offsets[min(e0 + base + i, e_end)];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int n = v[i + 1] - v[i];
      c[i] = n >= a.mfma_min ? (n + kBM - 1) / kBM : 0;  // experts with fewer tokens: the GEMV kernels
    }
  };
  int c[kPer];
  int cnt = 0;
  for (int base = 0; base < per; base += kPer) {
    counts(base, c);
#pragma unroll
    for (int i = 0; i < kPer; ++i) cnt += c[i];
  }
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  const int routed = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  if (t >= routed) {
    expert = -1;
    m0 = (t - routed) * kBM;
    return with_shared && a.T >= a.mfma_min && m0 < a.T;
  }
  const int owner = __ffsll((unsigned long long)__ballot(incl > t)) - 1;
  int local = t - (incl - cnt), e_hit = 0, m_hit = 0;
  for (int base = 0; base < per; base += kPer) {
    if (per > kPer) counts(base, c);  // one pass: the counts are still in registers
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (local >= 0 && local < c[i]) {
        e_hit = e0 + base + i;
        m_hit = local * kBM;
      }
      local -= c[i];
    }
  }
  // uniform values: the matrix bases derived from them stay in scalar registers
  expert = __builtin_amdgcn_readfirstlane(__shfl(e_hit, owner));
  m0 = __builtin_amdgcn_readfirstlane(__shfl(m_hit, owner));
  return true;
}

// NMAT = 2: gate and up (rows I, K = H), A = x gathered by token, epilogue
//           h = round_act(silu(g) u) into h (sorted order) / hs (shared).
// NMAT = 1: down (rows H, K = I), A = the expert's h rows, epilogue fp32 o / so.
// Block: 4 waves; wave w owns output rows nb + w * 16 WN + [0, 16 WN) and all
// 64 tokens of the tile (4 x WN MFMA tiles per matrix).
template <int QF, int NMAT, int WN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_expert_mfma(FfnArgs a, int with_shared, int n_blocks) {
  // one-dimensional grid, a multiple of 8 groups of kXcdTiles tiles: block b
  // runs on XCD b % 8; the work is dealt to the XCDs in groups of kXcdTiles
  // consecutive tiles (all their row slices), so a group's blocks share one L2
  // (the activation rows of a tile, the weights of an expert) and the groups
  // spread evenly over the XCDs.
  const int per_group = kXcdTiles * n_blocks;
  const int slot = (int)(blockIdx.x >> 3), xcd = (int)(blockIdx.x & 7);
  const int w = ((slot / per_group) * 8 + xcd) * per_group + slot % per_group;
  const int tile = w / n_blocks, nblk = w - tile * n_blocks;
  int expert, m0;
  if (!find_tile(a, with_shared != 0, tile, expert, m0)) return;
  const bool shared = expert < 0;
  const int lo = shared ? 0 : a.offsets[expert];
  const int n_rows = shared ? a.T : a.offsets[expert + 1] - lo;  // tokens of this expert
  const int kdim = NMAT == 2 ? a.H : a.I;   // reduction length
  const int rows = NMAT == 2 ? a.I : a.H;   // output rows per matrix
  const int G = kdim / kGroup;  // a multiple of kChunkG (checked by mfma_capable)
  const int nchunks = G / kChunkG;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, lc = lane >> 4;
  // ---- activations: the tile's 64 token rows by the DMA path, in the MFMA
  // fragment layout: fragment (M tile mt, group j of the chunk) is 1 KiB,
  // lane l holding row 16 mt + l % 16, elements 8 (l / 16) .. + 7 of the
  // group (raw bf16; the pair order of the codes is formed when read).  Wave
  // w copies the fragments of M tile w: its lanes' row (clamped to the
  // expert's last; such rows are dropped at the store).
  __shared__ __align__(16) uint8_t s_a0[16 * 1024];
  __shared__ __align__(16) uint8_t s_a1[16 * 1024];
  auto sa_of = [&](auto buf_c) -> uint8_t* {
    if constexpr (decltype(buf_c)::value == 0) return s_a0; else return s_a1;
  };
  const int rr = min(m0 + wave * 16 + ln, n_rows - 1);
  const uint16_t* arow;
  if constexpr (NMAT == 2) {
    const int tok = shared ? rr : a.sorted_pairs[lo + rr] / a.K;
    arow = reinterpret_cast<const uint16_t*>(a.x) + (size_t)tok * kdim;
  } else {
    arow = reinterpret_cast<const uint16_t*>(shared ? a.hs : a.h) + (size_t)(lo + rr) * kdim;
  }

  // ---- weights: the block's 256 row slots (NMAT x 64 WN rows) of codes and
  // scales (and minima) of one chunk, copied global -> LDS by the DMA path
  // (global_load_lds: lane i of an instruction lands at the wave-uniform LDS
  // base + 16 i or + 4 i), double buffered.  Slot s: matrix s / (64 WN), row
  // nblk * 64 WN + s % (64 WN) (clamped to the last row; never stored).
  //   4-bit codes: per 16 slots 1 KiB laid out [group q][slot][16 B]
  //   2-bit codes: per 32 slots 1 KiB laid out [group pair p][slot][16 B]
  //   3-bit codes: per 64 slots 3 KiB laid out [16-byte part q of the
  //                chunk's 48 bytes][slot][16 B]
  //   scales / minima: [slot][4 x fp16]
  // With these layouts the MFMA lanes' reads below hit 64 distinct banks; in
  // the 4-bit and 2-bit layouts every group of a chunk sits at a fixed
  // offset from one base address per lane.
  constexpr int kSlots = NMAT * 64 * WN;  // 256
  constexpr int kCodeChunk = kChunkG * code_bits(QF) * 4;  // code bytes per row per chunk: 64, 48, 32
  // one variable per buffer (the reads below are issued from asm, so the
  // compiler does not make them wait for the next chunk's copies)
  __shared__ __align__(16) uint8_t s_b0[kSlots * kCodeChunk];
  __shared__ __align__(16) uint8_t s_b1[kSlots * kCodeChunk];
  __shared__ __align__(16) uint16_t s_s0[kSlots * kChunkG];
  __shared__ __align__(16) uint16_t s_s1[kSlots * kChunkG];
  __shared__ __align__(16) uint16_t s_m0[QF == MOE_Q2_ASYM_G32 ? kSlots * kChunkG : 8];
  __shared__ __align__(16) uint16_t s_m1[QF == MOE_Q2_ASYM_G32 ? kSlots * kChunkG : 8];
  auto sb_of = [&](auto buf_c) -> uint8_t* {
    if constexpr (decltype(buf_c)::value == 0) return s_b0; else return s_b1;
  };
  auto ss_of = [&](auto buf_c) -> uint16_t* {
    if constexpr (decltype(buf_c)::value == 0) return s_s0; else return s_s1;
  };
  auto sm_of = [&](auto buf_c) -> uint16_t* {
    if constexpr (decltype(buf_c)::value == 0) return s_m0; else return s_m1;
  };
  const int eidx = shared ? 0 : expert;
  constexpr int kCodeBytesPerGroup = code_bits(QF) * 4;
  const uint32_t row_bytes = (uint32_t)G * kCodeBytesPerGroup;
  // the expert's matrices (uniform); pick field by field, since a reference
  // into the argument block would force it into scratch
  const uint8_t* cb[NMAT];
  const uint16_t* sb[NMAT];
  const uint16_t* mb[NMAT];
#pragma unroll
  for (int mi = 0; mi < NMAT; ++mi) {
    const uint8_t* codes;
    const uint16_t *scales, *mins;
    if (NMAT == 1) {
      codes = shared ? a.sdown.codes : a.down.codes;
      scales = shared ? a.sdown.scales : a.down.scales;
      mins = shared ? a.sdown.mins : a.down.mins;
    } else if (mi == 0) {
      codes = shared ? a.sgate.codes : a.gate.codes;
      scales = shared ? a.sgate.scales : a.gate.scales;
      mins = shared ? a.sgate.mins : a.gate.mins;
    } else {
      codes = shared ? a.sup.codes : a.up.codes;
      scales = shared ? a.sup.scales : a.up.scales;
      mins = shared ? a.sup.mins : a.up.mins;
    }
    cb[mi] = codes + (size_t)eidx * rows * row_bytes;
    sb[mi] = scales + (size_t)eidx * rows * G;
    mb[mi] = QF == MOE_Q2_ASYM_G32 ? mins + (size_t)eidx * rows * G : nullptr;
  }
  auto slot_row = [&](int slot) { return (uint32_t)min(nblk * 64 * WN + slot % (64 * WN), rows - 1); };
  // This wave's DMA sources: 4-bit codes, 4 instructions of 16 slots (lane ->
  // slot 16 i + lane % 16, group lane / 16); 3-bit codes, 3 of 64 slots
  // (instruction 3 w + i: slots 64 ((3 w + i) / 3) + lane, 16-byte part
  // (3 w + i) % 3); 2-bit codes, 2 of 32 slots (lane -> slot 32 i + lane % 32,
  // group pair lane / 32); scales (minima), 2 of 32 slots (lane -> slot
  // 32 i + lane / 2, group pair lane % 2).  Byte offsets within the chunk's
  // first group; matrix per instruction (uniform).
  constexpr int kCodeInst = code_bits(QF);
  uint32_t code_off[kCodeInst], scale_off[2];
#pragma unroll
  for (int i = 0; i < kCodeInst; ++i) {
    if constexpr (QF == MOE_Q4_SYM_G32) {
      const int slot = (wave * 4 + i) * 16 + (lane & 15);
      code_off[i] = slot_row(slot) * row_bytes + (uint32_t)(lane >> 4) * 16;
    } else if constexpr (QF == MOE_Q3_SYM_G32) {
      const int blk = wave * 3 + i;
      const int slot = (blk / 3) * 64 + lane;
      code_off[i] = slot_row(slot) * row_bytes + (uint32_t)(blk % 3) * 16;
    } else {
      const int slot = (wave * 2 + i) * 32 + (lane & 31);
      code_off[i] = slot_row(slot) * row_bytes + (uint32_t)(lane >> 5) * 16;
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int slot = (wave * 2 + i) * 32 + (lane >> 1);
    scale_off[i] = (slot_row(slot) * (uint32_t)G + (uint32_t)(lane & 1) * 2) * 2;  // bytes
  }
  auto dma = [&](int kc, auto buf_c, auto mta_c) {
    constexpr int MTA = decltype(mta_c)::value;
    if (wave < MTA) {  // this wave's M tile holds tokens: its four fragments of the chunk
#pragma unroll
      for (int j = 0; j < kChunkG; ++j)
        __builtin_amdgcn_global_load_lds(
            static_cast<const void*>(arow + (size_t)(kc * kChunkG + j) * kGroup + lc * 8),
            static_cast<void*>(sa_of(buf_c) + (wave * kChunkG + j) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kCodeInst; ++i) {
      const int blk = wave * kCodeInst + i;  // 1 KiB block of the chunk buffer
      const int mi = QF == MOE_Q3_SYM_G32 ? ((blk / 3) * 64) / (64 * WN)
                                          : (blk * (QF == MOE_Q4_SYM_G32 ? 16 : 32)) / (64 * WN);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(cb[mi] + code_off[i] + (uint32_t)kc * kCodeChunk),
                                       static_cast<void*>(sb_of(buf_c) + blk * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = wave * 2 + i;  // 32 slots x 8 bytes
      const int mi = (blk * 32) / (64 * WN);
      const uint32_t off = scale_off[i] + (uint32_t)kc * (kChunkG * 2);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(reinterpret_cast<const uint8_t*>(sb[mi]) + off),
                                       static_cast<void*>(ss_of(buf_c) + blk * 128), 4, 0, 0);
      if constexpr (QF == MOE_Q2_ASYM_G32)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(reinterpret_cast<const uint8_t*>(mb[mi]) + off),
                                         static_cast<void*>(sm_of(buf_c) + blk * 128), 4, 0, 0);
    }
  };

  // MFMA lanes: this wave's output rows nb + nt * 16 + ln of each matrix
  const int nb = nblk * (64 * WN) + wave * (16 * WN);
  auto slot_of = [&](int mi, int nt) { return mi * 64 * WN + wave * 16 * WN + nt * 16 + ln; };
  // a group's fp16 scale as fp32, converted by an instruction of its own (left
  // to the compiler, the conversion folds into a mixed-precision FMA per
  // product element; the same speed, but the 3-bit kernels then spill more)
  auto scale_f32 = [](uint2 v, int j) -> float {
    const uint32_t w = j < 2 ? v.x : v.y;
    const uint32_t h = (j & 1) ? (w >> 16) : w;
    float f;
    asm volatile("v_cvt_f32_f16 %0, %1" : "=v"(f) : "v"(h));
    return f;
  };
  auto half_of = [](uint2 v, int j) -> float {
    const uint32_t w = j < 2 ? v.x : v.y;
    return f16_to_f32((uint16_t)((j & 1) ? (w >> 16) : (w & 0xffffu)));
  };

  f32x4_t acc[NMAT][4][WN];
#pragma unroll
  for (int mi = 0; mi < NMAT; ++mi)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < WN; ++nt) acc[mi][mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr float kOff = QF == MOE_Q2_ASYM_G32 ? -1.0f : -1.5f;
  const uint32_t off2 = (uint32_t)(__float_as_uint(kOff) >> 16) * 0x10001u;  // two bf16 copies (exact)
  const uint32_t boff[4] = {off2, off2, off2, off2};
  auto compute = [&](auto buf_c, auto mta_c) {
    constexpr int MTA = decltype(mta_c)::value;  // active 16-row M tiles
    const uint8_t* sab = sa_of(buf_c);
    const uint8_t* sbb = sb_of(buf_c);
    static_assert(NMAT * WN == 4, "four (matrix, N tile) pairs per wave");
    uint2 sc4[NMAT][WN], mn4[NMAT][WN];
    {
      uint32_t as[4], am[4];
      uint2 rs[4], rm[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        as[p] = lds_addr(ss_of(buf_c) + slot_of(p / WN, p % WN) * kChunkG);
        am[p] = lds_addr(sm_of(buf_c) + (QF == MOE_Q2_ASYM_G32 ? slot_of(p / WN, p % WN) * kChunkG : 0));
      }
      lds_read4x2(as, rs);
      if constexpr (QF == MOE_Q2_ASYM_G32) lds_read4x2(am, rm);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        sc4[p / WN][p % WN] = rs[p];
        mn4[p / WN][p % WN] = QF == MOE_Q2_ASYM_G32 ? rm[p] : make_uint2(0u, 0u);
      }
    }
    // the groups' operands: four activation fragments and the four (matrix,
    // N tile) pairs' code dwords, one asm block per group; the fragments at
    // + 1024 j from one base, the 4-bit and 2-bit codes at + kBO from one
    // base per pair, the 3-bit codes (not at a fixed offset per group in
    // their layout) from addresses of their own
    constexpr int kNB = QF == MOE_Q3_SYM_G32 ? 8 : 4;
    const uint32_t abase = lds_addr(sab + lane * 16);
    uint32_t cbase[kNB];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int slot = slot_of(p / WN, p % WN);
      if constexpr (QF == MOE_Q4_SYM_G32) {
        cbase[p] = lds_addr(&sbb[(slot >> 4) * 1024 + (slot & 15) * 16 + lc * 4]);
      } else if constexpr (QF == MOE_Q2_ASYM_G32) {
        cbase[p] = lds_addr(&sbb[(slot >> 5) * 1024 + (slot & 31) * 16 + (lc >> 1) * 4]);
      }
    }
    auto group = [&](auto j_c) {
      constexpr int j = decltype(j_c)::value;
      constexpr int kBO = QF == MOE_Q4_SYM_G32 ? j * 256 : QF == MOE_Q2_ASYM_G32 ? (j >> 1) * 512 + (j & 1) * 8 : 0;
      if constexpr (QF == MOE_Q3_SYM_G32) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          // the lane's 8 codes: low-bit bytes 12 j + 2 lc, + 1 and third-bit byte 12 j + 8 + lc of the chunk
          const int slot = slot_of(p / WN, p % WN);
          const uint8_t* base = &sbb[(slot >> 6) * 3072 + (slot & 63) * 16];
          const int o1 = 12 * j + 2 * lc, o2 = 12 * j + 8 + lc;
          cbase[p] = lds_addr(base + (o1 >> 4) * 1024 + (o1 & 12));      // the dword holding bytes o1, o1 + 1
          cbase[4 + p] = lds_addr(base + (o2 >> 4) * 1024 + (o2 & 12));  // the dword holding byte o2
        }
      }
      frag4_t fr[4];
      uint32_t cw[kNB];
      grp_read<kNB, j * 1024, kBO, kBO>(abase, cbase, fr, cw);
      uint32_t af[4][4];
      f32x4_t cf[4];
      uint32_t bw[NMAT][WN];
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) {
        // (x0..x7) -> pairs (x0,x4) (x1,x5) (x2,x6) (x3,x7), the codes' order;
        // one byte permute each (bytes 0-3 of the selector's space are the
        // second operand's, 4-7 the first's)
        af[mt][0] = __builtin_amdgcn_perm(fr[mt][2], fr[mt][0], 0x05040100u);
        af[mt][1] = __builtin_amdgcn_perm(fr[mt][2], fr[mt][0], 0x07060302u);
        af[mt][2] = __builtin_amdgcn_perm(fr[mt][3], fr[mt][1], 0x05040100u);
        af[mt][3] = __builtin_amdgcn_perm(fr[mt][3], fr[mt][1], 0x07060302u);
        cf[mt] = mfma16(af[mt], boff, f32x4_t{0.f, 0.f, 0.f, 0.f});  // the offset term of each token
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t v;
        if constexpr (QF == MOE_Q4_SYM_G32) {
          v = cw[p];
        } else if constexpr (QF == MOE_Q3_SYM_G32) {
          v = ((cw[p] >> ((lc & 1) * 16)) & 0xffffu) | (((cw[4 + p] >> (lc * 8)) & 0xffu) << 16);
        } else {
          v = (cw[p] >> ((lc & 1) * 16)) & 0xffffu;
        }
        bw[p / WN][p % WN] = v;
      }
      // software pipeline over the NW (matrix, N tile) pairs: the products of
      // pair p are issued before the scaling of pair p - 1
      constexpr int NW = NMAT * WN;
      f32x4_t dp[4];
      float scp = 0.f, mnp = 0.f;
#pragma unroll
      for (int p = 0; p <= NW; ++p) {
        f32x4_t dc[4];
        float scc = 0.f, mnc = 0.f;
        if (p < NW) {
          const int mi = p / WN, nt = p % WN;
          uint32_t bf[4];
          unpack_b<QF>(bw[mi][nt], bf);
          scc = scale_f32(sc4[mi][nt], j);
          if constexpr (QF == MOE_Q2_ASYM_G32) mnc = half_of(mn4[mi][nt], j) * -0.25f;
#pragma unroll
          for (int mt = 0; mt < MTA; ++mt) dc[mt] = mfma16(af[mt], bf, cf[mt]);
        }
        if (p > 0) {
          const int mi = (p - 1) / WN, nt = (p - 1) % WN;
#pragma unroll
          for (int mt = 0; mt < MTA; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mi][mt][nt][i] = fmaf(scp, dp[mt][i], acc[mi][mt][nt][i]);
            if constexpr (QF == MOE_Q2_ASYM_G32) {
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[mi][mt][nt][i] = fmaf(mnp, cf[mt][i], acc[mi][mt][nt][i]);
            }
          }
        }
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt) dp[mt] = dc[mt];
        scp = scc;
        mnp = mnc;
      }
#pragma unroll
      for (int mi = 0; mi < NMAT; ++mi)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < WN; ++nt) asm volatile("" : "+v"(acc[mi][mt][nt]));
      // (the empty asm statements above keep each product's scaling next to
      // it: left alone, the compiler sinks the scaling past later groups'
      // products and holds every product's result at once)
      __builtin_amdgcn_sched_barrier(0);
    };
    group(std::integral_constant<int, 0>{});
    group(std::integral_constant<int, 1>{});
    group(std::integral_constant<int, 2>{});
    group(std::integral_constant<int, 3>{});
    static_assert(kChunkG == 4, "four groups per chunk");
  };

  // the DMA writes LDS behind the compiler's back: wait for it (vmcnt) with a
  // memory clobber before the barrier that publishes the chunk
  auto wait_dma = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // one chunk in buffer BUF while the next one is copied into the other
  auto step = [&](int kc, auto buf_c, auto mta_c) {
    constexpr int buf = decltype(buf_c)::value;
    if (kc + 1 < nchunks) dma(kc + 1, std::integral_constant<int, buf ^ 1>{}, mta_c);
    compute(buf_c, mta_c);
    wait_dma();
    __syncthreads();
  };
  // the chunk loop, two chunks per pass (buffers 0 and 1), specialised by the
  // number of 16-row M tiles that hold tokens of the expert (a partial tile
  // skips the copies and products of its empty ones)
  auto chunks = [&](auto mta_c) {
    dma(0, B0{}, mta_c);
    wait_dma();
    __syncthreads();
    for (int kc = 0; kc < nchunks; kc += 2) {
      step(kc, B0{}, mta_c);
      if (kc + 1 < nchunks) step(kc + 1, B1{}, mta_c);
    }
  };
  const int mt_act = min(4, (n_rows - m0 + 15) / 16);  // uniform
  if (mt_act <= 1) chunks(std::integral_constant<int, 1>{});
  else if (mt_act == 2) chunks(std::integral_constant<int, 2>{});
  else if (mt_act == 3) chunks(std::integral_constant<int, 3>{});
  else chunks(std::integral_constant<int, 4>{});

  // ---- epilogue: D lane l holds token rows 4 (l / 16) + i of each M tile, column ln
  constexpr float kUnit = QF == MOE_Q4_SYM_G32 ? 16.f : QF == MOE_Q3_SYM_G32 ? 8.f : 4.f;  // the codes' 1/16, 1/8, 1/4
  const bool all_rows = (nblk + 1) * (64 * WN) <= rows;  // uniform: no row of this block is past the end
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + mt * 16 + lc * 4 + i;
      if (m >= n_rows) continue;
      const size_t orow = shared ? (size_t)m : (size_t)(lo + m);
      if constexpr (NMAT == 2) {
        uint16_t* hrow = reinterpret_cast<uint16_t*>(shared ? a.hs : a.h) + orow * rows;
#pragma unroll
        for (int nt = 0; nt < WN; ++nt) {
          const int n = nb + nt * 16 + ln;
          if (all_rows || n < rows) {
            const float g = acc[0][mt][nt][i] * kUnit, u = acc[1][mt][nt][i] * kUnit;
            // silu(g) = g / (1 + e^-g), the quotient as a product with the
            // hardware reciprocal (within 2 ulp: far below the bf16 rounding)
            const float sg = g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.44269504088896341f));
            hrow[n] = f32_to_bf16(sg * u);
          }
        }
      } else {
        float* orow_p = (shared ? a.so : a.o) + orow * rows;
#pragma unroll
        for (int nt = 0; nt < WN; ++nt) {
          const int n = nb + nt * 16 + ln;
          if (all_rows || n < rows) orow_p[n] = acc[0][mt][nt][i] * kUnit;
        }
      }
    }
}

// Upper bound of the tile count: sum over the experts with n_e >= mfma_min of
// ceil(n_e / 64) <= T K / 64 + min(E, T K / mfma_min), plus the shared tiles.
static int tile_capacity(const FfnArgs& a, bool with_shared) {
  const int64_t pairs = (int64_t)a.T * a.K;
  const int64_t hot = pairs / (a.mfma_min > 1 ? a.mfma_min : 1);
  return (int)(pairs / kBM + (hot < a.E ? hot : a.E) +
               (with_shared && a.T >= a.mfma_min ? (a.T + kBM - 1) / kBM : 0));
}

// Matrix-core path: bf16 activations (the A operand is the activation
// itself), on average at least 8 tokens per expert, H and I multiples of 128
// (whole chunks of 4 groups) and 8-byte aligned scale and minimum arrays.
static bool al8(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 7) == 0; }
static bool qm_al8(const QMat& q) { return al8(q.scales) && al8(q.mins); }

static bool mfma_capable(const FfnArgs& a) {
  const int chunk = kGroup * kChunkG;
  return a.act == MOE_ACT_BF16 && a.H % chunk == 0 && a.I % chunk == 0 && qm_al8(a.gate) && qm_al8(a.up) &&
         qm_al8(a.down) && (!a.n_shared || (qm_al8(a.sgate) && qm_al8(a.sup) && qm_al8(a.sdown)));
}

// The expert split for T tokens (FfnArgs::mfma_min): every expert on the
// grouped GEMM from 8 tokens per expert on average; below that, past the
// small-batch pair count, only the experts with at least kHotTokens tokens
// (under the router's skew a few experts take most of the tokens: a GEMV
// block row would walk them a few tokens at a time); none for fewer pairs.
constexpr int kHotTokens = 8;
constexpr int kSplitMinPairs = 256;
int mfma_split(const FfnArgs& a) {
  if (!mfma_capable(a)) return 0;
  const int64_t pairs = (int64_t)a.T * a.K;
  if (pairs >= 8 * (int64_t)a.E) return 1;
  if (pairs > kSplitMinPairs) return 1;
  return 0;
}

hipError_t launch_mfma_gateup(const FfnArgs& a, hipStream_t s) {
  const bool ws = a.n_shared && a.hs;
  const int nb = (a.I + 127) / 128;  // 4 waves x 2 N tiles of 16 rows of I
  const int64_t unit = (int64_t)8 * kXcdTiles * nb;
  const dim3 grid((unsigned)(((int64_t)nb * tile_capacity(a, ws) + unit - 1) / unit * unit));
  by_qfmt(a.qfmt, [&](auto q) { k_expert_mfma<decltype(q)::value, 2, 2><<<grid, 256, 0, s>>>(a, ws, nb); });
  return hipGetLastError();
}

hipError_t launch_mfma_down(const FfnArgs& a, hipStream_t s) {
  const bool ws = a.n_shared && a.so;
  const int nb = (a.H + 255) / 256;  // 4 waves x 4 N tiles of 16 rows of H
  const int64_t unit = (int64_t)8 * kXcdTiles * nb;
  const dim3 grid((unsigned)(((int64_t)nb * tile_capacity(a, ws) + unit - 1) / unit * unit));
  by_qfmt(a.qfmt, [&](auto q) { k_expert_mfma<decltype(q)::value, 1, 4><<<grid, 256, 0, s>>>(a, ws, nb); });
  return hipGetLastError();
}

}  // namespace moe
