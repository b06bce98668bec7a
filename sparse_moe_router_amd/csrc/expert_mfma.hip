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
// 1 + u / 16 (4-bit) or 1 + u / 4 (2-bit); with bf16 x every product is exact
// in fp32, and the offset term enters through the MFMA's accumulator input:
//   4-bit:  D = sum (1 + u/16) x - 1.5 sum x = sum (u - 8) x / 16,  acc += 16 s D
//   2-bit:  D = sum (1 + u/4) x - sum x      = sum u x / 4,         acc += 4 s D + m sum x
// Keeping the code in the top mantissa bits keeps the cancelled offset within
// a few times the signal, so the fp32 sums lose little to the cancellation.
// The offset sum x is computed once per (token, group) while the activations
// are staged in LDS.
//
// v_mfma_f32_16x16x32_bf16 lane layout (gfx950): A lane l holds row l % 16,
// k = 8 (l / 16) .. + 7; B lane l holds column l % 16 at the same k; D lane l
// holds rows 4 (l / 16) + i, column l % 16.  The codes of one B lane are 8
// consecutive codes and are unpacked into the pairs (k_j, k_{j+4}); the
// activations are stored in LDS in that same pair order.
#include "gemv_tile.h"
#include <type_traits>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;          // tokens per tile
constexpr int kXcdTiles = 4;     // tiles per XCD work group
constexpr int kChunkG = 4;       // groups (of 32 k) per staged chunk
constexpr int kRowWords = kChunkG * 16 + 4;  // LDS words per token row per chunk (+4 pad: no bank conflicts)

__device__ __forceinline__ f32x4_t mfma16(const uint32_t (&a)[4], const uint32_t (&b)[4], f32x4_t c) {
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v av = {a[0], a[1], a[2], a[3]};
  const u32x4v bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                 c, 0, 0, 0);
}

// 8 codes of one B lane -> 4 bf16 pairs (k_j, k_{j+4}): 1 + u/16 (4-bit) or 1 + u/4 (2-bit).
template <int QF>
__device__ __forceinline__ void unpack_b(uint32_t w, uint32_t (&b)[4]) {
  asm volatile("" : "+v"(w));  // unpack at the point of use
  if constexpr (QF == MOE_Q4_SYM_G32) {  // nibble j -> bits 3..6, nibble j + 4 -> bits 19..22
    b[0] = and_or(w << 3, 0x00780078u, 0x3f803f80u);
    b[1] = and_or(w >> 1, 0x00780078u, 0x3f803f80u);
    b[2] = and_or(w >> 5, 0x00780078u, 0x3f803f80u);
    b[3] = and_or(w >> 9, 0x00780078u, 0x3f803f80u);
  } else {  // 16 bits = 8 crumbs; the second byte moves to bits 16..23, crumb j -> bits 5..6
    const uint32_t s = (w & 0xffu) | ((w & 0xff00u) << 8);
    b[0] = and_or(s << 5, 0x00600060u, 0x3f803f80u);
    b[1] = and_or(s << 3, 0x00600060u, 0x3f803f80u);
    b[2] = and_or(s << 1, 0x00600060u, 0x3f803f80u);
    b[3] = and_or(s >> 1, 0x00600060u, 0x3f803f80u);
  }
}

// Work tiles: ceil(n_e / 64) per routed expert in expert order, then
// ceil(T / 64) for the shared expert.  Every wave of a block derives its tile
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
    for (int i = 0; i < kPer; ++i) c[i] = (v[i + 1] - v[i] + kBM - 1) / kBM;
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
    return with_shared && m0 < a.T;
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
  const int G = kdim / kGroup;  // a multiple of kChunkG (checked by mfma_ok)
  const int nchunks = G / kChunkG;

  __shared__ __align__(16) uint32_t s_a[2][kBM * kRowWords];
  __shared__ __align__(16) float s_c[2][kChunkG][kBM];  // offset term per (group, token)

  // ---- staging role: thread -> (token row r, group jg of the chunk)
  const int r = threadIdx.x >> 2, jg = threadIdx.x & 3;
  const int rr = min(m0 + r, n_rows - 1);  // clamped: rows past the expert's end are dropped at the store
  const uint16_t* arow;
  if constexpr (NMAT == 2) {
    const int tok = shared ? rr : a.sorted_pairs[lo + rr] / a.K;
    arow = reinterpret_cast<const uint16_t*>(a.x) + (size_t)tok * kdim;
  } else {
    arow = reinterpret_cast<const uint16_t*>(shared ? a.hs : a.h) + (size_t)(lo + rr) * kdim;
  }
  uint4 stage[4];
  auto load_a = [&](int kc) {
    const int g = kc * kChunkG + jg;
    const uint4* src = reinterpret_cast<const uint4*>(arow + (size_t)g * kGroup);
#pragma unroll
    for (int i = 0; i < 4; ++i) stage[i] = src[i];
  };
  auto store_a = [&](int buf) {
    uint32_t* dst = &s_a[buf][r * kRowWords + jg * 16];
    float sx0 = 0.f, sx1 = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // chunk of 8: (x0..x7) -> pairs (x0,x4) (x1,x5) (x2,x6) (x3,x7)
      const uint4 q = stage[c];
      uint4 p;
      p.x = (q.x & 0xffffu) | (q.z << 16);
      p.y = (q.x >> 16) | (q.z & 0xffff0000u);
      p.z = (q.y & 0xffffu) | (q.w << 16);
      p.w = (q.y >> 16) | (q.w & 0xffff0000u);
      *reinterpret_cast<uint4*>(dst + 4 * c) = p;
      sx0 = dot2_bf16(0x3f803f80u, p.x, sx0);
      sx1 = dot2_bf16(0x3f803f80u, p.y, sx1);
      sx0 = dot2_bf16(0x3f803f80u, p.z, sx0);
      sx1 = dot2_bf16(0x3f803f80u, p.w, sx1);
    }
    const float sx = sx0 + sx1;
    s_c[buf][jg][r] = QF == MOE_Q4_SYM_G32 ? -1.5f * sx : -sx;
  };

  // ---- weights: the block's 256 row slots (NMAT x 64 WN rows) of codes and
  // scales (and minima) of one chunk, copied global -> LDS by the DMA path
  // (global_load_lds: lane i of an instruction lands at the wave-uniform LDS
  // base + 16 i or + 4 i), double buffered.  Slot s: matrix s / (64 WN), row
  // nblk * 64 WN + s % (64 WN) (clamped to the last row; never stored).
  //   4-bit codes: per 16 slots 1 KiB laid out [group q][slot][16 B]
  //   2-bit codes: per 32 slots 1 KiB laid out [group pair p][slot][16 B]
  //   scales / minima: [slot][4 x fp16]
  // With these layouts the MFMA lanes' reads below hit 64 distinct banks.
  constexpr int kSlots = NMAT * 64 * WN;  // 256
  constexpr int kCodeChunk = QF == MOE_Q4_SYM_G32 ? 64 : 32;  // code bytes per row per chunk
  __shared__ __align__(16) uint8_t s_b[2][kSlots * kCodeChunk];
  __shared__ __align__(16) uint16_t s_s[2][kSlots * kChunkG];
  __shared__ __align__(16) uint16_t s_m[QF == MOE_Q2_ASYM_G32 ? 2 : 1][QF == MOE_Q2_ASYM_G32 ? kSlots * kChunkG : 8];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 15, lc = lane >> 4;
  const int eidx = shared ? 0 : expert;
  constexpr int kCodeBytesPerGroup = QF == MOE_Q4_SYM_G32 ? 16 : 8;
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
  // slot 16 i + lane % 16, group lane / 16); 2-bit codes, 2 of 32 slots (lane
  // -> slot 32 i + lane % 32, group pair lane / 32); scales (minima), 2 of 32
  // slots (lane -> slot 32 i + lane / 2, group pair lane % 2).  Byte offsets
  // within the chunk's first group; matrix per instruction (uniform).
  constexpr int kCodeInst = QF == MOE_Q4_SYM_G32 ? 4 : 2;
  uint32_t code_off[kCodeInst], scale_off[2];
#pragma unroll
  for (int i = 0; i < kCodeInst; ++i) {
    if constexpr (QF == MOE_Q4_SYM_G32) {
      const int slot = (wave * 4 + i) * 16 + (lane & 15);
      code_off[i] = slot_row(slot) * row_bytes + (uint32_t)(lane >> 4) * 16;
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
  auto dma_b = [&](int kc, int buf) {
#pragma unroll
    for (int i = 0; i < kCodeInst; ++i) {
      const int blk = wave * kCodeInst + i;  // 1 KiB block of the chunk buffer
      const int mi = (blk * (QF == MOE_Q4_SYM_G32 ? 16 : 32)) / (64 * WN);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(cb[mi] + code_off[i] + (uint32_t)kc * kCodeChunk),
                                       static_cast<void*>(&s_b[buf][blk * 1024]), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = wave * 2 + i;  // 32 slots x 8 bytes
      const int mi = (blk * 32) / (64 * WN);
      const uint32_t off = scale_off[i] + (uint32_t)kc * (kChunkG * 2);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(reinterpret_cast<const uint8_t*>(sb[mi]) + off),
                                       static_cast<void*>(&s_s[buf][blk * 128]), 4, 0, 0);
      if constexpr (QF == MOE_Q2_ASYM_G32)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(reinterpret_cast<const uint8_t*>(mb[mi]) + off),
                                         static_cast<void*>(&s_m[buf][blk * 128]), 4, 0, 0);
    }
  };

  // MFMA lanes: this wave's output rows nb + nt * 16 + ln of each matrix
  const int nb = nblk * (64 * WN) + wave * (16 * WN);
  auto slot_of = [&](int mi, int nt) { return mi * 64 * WN + wave * 16 * WN + nt * 16 + ln; };
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

  auto compute = [&](int buf, auto mta_c) {
    constexpr int MTA = decltype(mta_c)::value;  // active 16-row M tiles
    uint2 sc4[NMAT][WN], mn4[NMAT][WN];
#pragma unroll
    for (int mi = 0; mi < NMAT; ++mi)
#pragma unroll
      for (int nt = 0; nt < WN; ++nt) {
        sc4[mi][nt] = *reinterpret_cast<const uint2*>(&s_s[buf][slot_of(mi, nt) * kChunkG]);
        if constexpr (QF == MOE_Q2_ASYM_G32) mn4[mi][nt] = *reinterpret_cast<const uint2*>(&s_m[buf][slot_of(mi, nt) * kChunkG]);
      }
    struct GroupOps {
      uint32_t af[4][4];
      f32x4_t cf[4];
      uint32_t bw[NMAT][WN];
    };
    auto lds_group = [&](int j, GroupOps& g) {
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) {
        const uint4 v = *reinterpret_cast<const uint4*>(&s_a[buf][(mt * 16 + ln) * kRowWords + j * 16 + lc * 4]);
        g.af[mt][0] = v.x; g.af[mt][1] = v.y; g.af[mt][2] = v.z; g.af[mt][3] = v.w;
        g.cf[mt] = *reinterpret_cast<const f32x4_t*>(&s_c[buf][j][mt * 16 + lc * 4]);
      }
#pragma unroll
      for (int mi = 0; mi < NMAT; ++mi)
#pragma unroll
        for (int nt = 0; nt < WN; ++nt) {
          const int slot = slot_of(mi, nt);
          if constexpr (QF == MOE_Q4_SYM_G32) {
            g.bw[mi][nt] = *reinterpret_cast<const uint32_t*>(&s_b[buf][(slot >> 4) * 1024 + j * 256 + (slot & 15) * 16 + lc * 4]);
          } else {
            g.bw[mi][nt] = *reinterpret_cast<const uint16_t*>(
                &s_b[buf][(slot >> 5) * 1024 + (j >> 1) * 512 + (slot & 31) * 16 + (j & 1) * 8 + lc * 2]);
          }
        }
    };
    GroupOps gops[2];
    lds_group(0, gops[0]);
#pragma unroll
    for (int j = 0; j < kChunkG; ++j) {
      if (j + 1 < kChunkG) lds_group(j + 1, gops[(j + 1) & 1]);  // next group's operands in flight
      auto& af = gops[j & 1].af;
      auto& cf = gops[j & 1].cf;
      auto& bw = gops[j & 1].bw;
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
          scc = half_of(sc4[mi][nt], j);
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
    }
  };

  // the DMA writes LDS behind the compiler's back: wait for it (vmcnt) with a
  // memory clobber before the barrier that publishes the chunk
  auto wait_dma = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  dma_b(0, 0);
  load_a(0);
  store_a(0);
  wait_dma();
  __syncthreads();
  // the chunk loop, specialised by the number of 16-row M tiles that hold
  // tokens of the expert (a partial tile skips the products of its empty ones)
  auto chunks = [&](auto mta_c) {
    for (int kc = 0; kc < nchunks; ++kc) {
      const int buf = kc & 1;
      const bool more = kc + 1 < nchunks;
      if (more) {
        dma_b(kc + 1, buf ^ 1);
        load_a(kc + 1);
      }
      compute(buf, mta_c);
      if (more) store_a(buf ^ 1);
      wait_dma();
      __syncthreads();
    }
  };
  const int mt_act = min(4, (n_rows - m0 + 15) / 16);  // uniform
  if (mt_act <= 1) chunks(std::integral_constant<int, 1>{});
  else if (mt_act == 2) chunks(std::integral_constant<int, 2>{});
  else if (mt_act == 3) chunks(std::integral_constant<int, 3>{});
  else chunks(std::integral_constant<int, 4>{});

  // ---- epilogue: D lane l holds token rows 4 (l / 16) + i of each M tile, column ln
  constexpr float kUnit = QF == MOE_Q4_SYM_G32 ? 16.f : 4.f;  // the codes' 1/16 or 1/4, exactly
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

// Upper bound of the tile count: sum_e ceil(n_e / 64) <= T K / 64 + (experts hit).
static int tile_capacity(const FfnArgs& a, bool with_shared) {
  const int64_t pairs = (int64_t)a.T * a.K;
  return (int)(pairs / kBM + (pairs < a.E ? pairs : a.E) + (with_shared ? (a.T + kBM - 1) / kBM : 0));
}

// Matrix-core path: bf16 activations (the A operand is the activation
// itself), on average at least 8 tokens per expert, H and I multiples of 128
// (whole chunks of 4 groups) and 8-byte aligned scale and minimum arrays.
static bool al8(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 7) == 0; }
static bool qm_al8(const QMat& q) { return al8(q.scales) && al8(q.mins); }

bool mfma_ok(const FfnArgs& a) {
  const int chunk = kGroup * kChunkG;
  return a.act == MOE_ACT_BF16 && (int64_t)a.T * a.K >= 8 * (int64_t)a.E && a.H % chunk == 0 && a.I % chunk == 0 &&
         qm_al8(a.gate) && qm_al8(a.up) && qm_al8(a.down) && (!a.n_shared || (qm_al8(a.sgate) && qm_al8(a.sup) &&
                                                                               qm_al8(a.sdown)));
}

hipError_t launch_mfma_gateup(const FfnArgs& a, hipStream_t s) {
  const bool ws = a.n_shared && a.hs;
  const int nb = (a.I + 127) / 128;  // 4 waves x 2 N tiles of 16 rows of I
  const int64_t unit = (int64_t)8 * kXcdTiles * nb;
  const dim3 grid((unsigned)(((int64_t)nb * tile_capacity(a, ws) + unit - 1) / unit * unit));
  if (a.qfmt == MOE_Q4_SYM_G32) k_expert_mfma<MOE_Q4_SYM_G32, 2, 2><<<grid, 256, 0, s>>>(a, ws, nb);
  else k_expert_mfma<MOE_Q2_ASYM_G32, 2, 2><<<grid, 256, 0, s>>>(a, ws, nb);
  return hipGetLastError();
}

hipError_t launch_mfma_down(const FfnArgs& a, hipStream_t s) {
  const bool ws = a.n_shared && a.so;
  const int nb = (a.H + 255) / 256;  // 4 waves x 4 N tiles of 16 rows of H
  const int64_t unit = (int64_t)8 * kXcdTiles * nb;
  const dim3 grid((unsigned)(((int64_t)nb * tile_capacity(a, ws) + unit - 1) / unit * unit));
  if (a.qfmt == MOE_Q4_SYM_G32) k_expert_mfma<MOE_Q4_SYM_G32, 1, 4><<<grid, 256, 0, s>>>(a, ws, nb);
  else k_expert_mfma<MOE_Q2_ASYM_G32, 1, 4><<<grid, 256, 0, s>>>(a, ws, nb);
  return hipGetLastError();
}

}  // namespace moe
