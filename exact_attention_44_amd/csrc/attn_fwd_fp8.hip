// attn_fwd_fp8.hip - fused attention forward over 8-bit floating-point inputs
// for gfx950 (CDNA4), and its C ABI.
//
// Method: the same tiled walk with online softmax as the bf16 forward
// (news.hamidun.com glossary "Flash attention", second paragraph; onecalc.app
// "Attention memory", section "FlashAttention"). The glossary's second
// paragraph names FP8 precision as the third version's addition. Here Q, K and
// V arrive as OCP E4M3 codes with one float32 descale factor per (batch item,
// head) each, both products run on the 8-bit matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, float32 accumulation), and the softmax weights
// are rounded to E4M3 for the value product. The running max, row sums and
// the output accumulator stay float32; the output is bf16.
//
// Decomposition and schedule follow the bf16 kernel: one workgroup per
// (b, h, 256 query rows), 8 waves of 32 rows, waves w and w + 4 on one SIMD,
// the two groups of four alternating matrix steps (value product of the
// previous tile, score product of this one) and vector steps (masks and
// softmax), one workgroup barrier per key tile.
//
// Operand layouts. Scores are computed transposed, S^T = K Q^T: A = 32 keys x
// 64 features (K rows in their natural order), B = 64 features x 32 queries
// (Q in registers). In the 32x32 accumulator lane L holds query L % 32 and the
// 16 keys 8a + 4h + b (a, b in 0..3, h = L / 32) of each 32-key block. The
// value product O^T += V^T P^T takes a whole 64-key tile in one k-step: the
// B operand is lane L's 32 weights, byte j = register j % 16 of key block
// j / 16, so slot (h, j) of the k axis is key
//   key(h, j) = 32 (j / 16) + 8 ((j % 16) / 4) + 4 h + j % 4,
// and the A operand (V^T: 32 feature rows x the same 64 key slots) is read
// from the row-major V tile with LDS transpose reads that gather, for each
// lane's feature, the bytes of exactly those keys.
//
// LDS per tile: K row-major in key order, V row-major in k-slot order (LDS row
// 32 h + j holds key(h, j), so each transpose read covers eight consecutive
// rows), both with unpadded D-byte rows whose 16-byte slots are permuted by an
// XOR with a function of the row (k_swz, v_swz) chosen so that every fragment
// read hits distinct banks. Both tiles arrive by buffer loads that write LDS
// directly; a half tile is a whole number of 64-slot load instructions, so
// every wave issues the same loads.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "attn.h"
#include "attn_common.h"

namespace {

using namespace attn_detail;

struct Fp8Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* dsq;  // descale factors [B*H] or null (1)
  const float* dsk;
  const float* dsv;
  uint16_t* out;
  float* lse;
  const uint8_t* kpm;
  int s_q, s_k, H, BH, n_qt;
  int n_items;      // work items: query tiles x (b, h)
  float scale;
};

// XOR applied to the 16-byte slot index of K row r. A score-product fragment
// read covers 16 consecutive rows at one logical slot; with D-byte rows the
// bank group of (row, slot) is (r * D / 16 + slot) mod 16, and the XOR makes
// the 16 rows' groups distinct.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

// XOR applied to the 16-byte slot index of V's LDS row r. A transpose read
// covers eight consecutive rows at two adjacent slots per lane half; the XOR
// (which keeps the low bit of the slot) makes their 16 bank groups distinct.
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? 2 * ((r >> 1) & 3) : 2 * ((r >> 2) & 1);
}

// Key (within the 64-key tile) at slot j of lane half h of the value
// product's k axis: the key that score accumulator register j % 16 of key
// block j / 16 holds in that lane half.
__device__ __forceinline__ int key_of_slot(int h, int j) {
  return 32 * (j >> 4) + 8 * ((j & 15) >> 2) + 4 * h + (j & 3);
}

template <int D, bool CAUSAL, bool PADMASK>
__global__ __launch_bounds__(512, 2) void attn_fwd_fp8_kernel(Fp8Params p) {
  constexpr int NT = 512;             // 8 waves: two ping-pong groups of 4
  constexpr int BR = 256;             // query rows per workgroup, 32 per wave
  constexpr int BC = 64;              // keys per tile (one k-step of the value product)
  constexpr int KB = BC / 32;         // 32-key blocks of the score tile
  constexpr int DK = D / 64;          // k-steps of the score product
  constexpr int DB = D / 32;          // 32-feature blocks of the output
  constexpr int KU = D / 16;          // 16-byte units per K or V row
  constexpr int K_BYTES = BC * D;
  constexpr int V_BYTES = BC * D;
  constexpr int BUF_BYTES = K_BYTES + V_BYTES;
  constexpr int NBUF = 4;
  // Each group stages half of a tile's LDS rows: K rows 32 grp .. +31 (keys
  // 32 grp ..) and V rows 32 grp .. +31 (the keys of lane half grp), each
  // 32 rows of KU 16-byte slots written by DMA instructions of 64 consecutive
  // LDS slots; each lane loads the memory slot that belongs in its LDS slot.
  constexpr int H_SLOTS = 32 * KU;
  constexpr int N_DMA = H_SLOTS / 64;  // per half tile, of K and of V
  static_assert(H_SLOTS % 64 == 0 && N_DMA <= 4, "a half tile is at most one DMA per wave");
  // Weights are taken against a reference max that can lag the true one;
  // their float32 tile sum bounds every weight, and E4M3 conversion turns
  // magnitudes from 480 up into NaN, so a tile whose sum exceeds 256 is
  // recomputed against the true max (see finish()).
  constexpr float kSumLimit = 256.f;

  __shared__ __attribute__((aligned(16))) char lds[NBUF * BUF_BYTES];
  __shared__ int lds_last;
  // With a padding mask: the key tiles of the current item that hold a
  // visible key, in order (see build_tile_list); items with more tiles than
  // the list holds walk every tile up to the last unpadded key.
  __shared__ uint16_t lds_tl[PADMASK ? kTileListMax + 8 : 1];
  __shared__ __attribute__((aligned(8))) uint8_t lds_bits[PADMASK ? kTileListMax / 8 : 8];
  __shared__ int lds_scr[3 * (NT / 64) + 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv >> 2;
  const int hl = lane >> 5;
  const int ln = lane & 31;

  const int s_q = p.s_q, s_k = p.s_k;
  // ---- work items (query tile, (b, h)), (b, h) fastest, the longest causal
  // tiles first. At D = 128 each workgroup takes one item (L = its index); at
  // D = 64 the grid is persistent (at most one workgroup per CU) and
  // workgroup g takes item g in even rounds and its mirror image within the
  // round (keeping g mod 8) in odd rounds, as the bf16 kernel does.
  constexpr bool PERSIST = D == 64;
  const int G = gridDim.x, g = blockIdx.x;
  auto item_of = [&](int round) -> int {
    const int off = (round & 1) ? ((G & 7) == 0 ? G - 8 * (1 + g / 8) + (g & 7) : G - 1 - g) : g;
    return round * G + off;
  };
  int round = 0;
  int L_cur = item_of(0);  // < n_items: the grid is at most the item count
  int boff = 0;            // LDS buffer of the item's tile t: (boff + t) % NBUF
  // per-item values (workgroup-uniform)
  int bh = 0, b = 0, q0 = 0, qlo = 0, n_kv = 0;
  float dv = 1.f, c = kLog2e, scale_abs = 0.f;
  uint32_t q_and = ~0u, q_xor = 0u;
  const uint8_t* kg = nullptr;
  const uint8_t* vg = nullptr;
  const uint8_t* mg = nullptr;
  i32x8_t qf[DK];

  // ---- staging of this group's half (keys 32 grp .. 32 grp + 31) of a tile
  const int wg = wv & 3;  // this wave's DMA instruction within its group's half
  uint32_t k_voff, v_voff;
  {
    const int slot = 64 * wg + lane;  // LDS slot within the half tile
    const int r = slot / KU, ph = slot % KU;
    k_voff = (uint32_t)((32 * grp + r) * D + 16 * (ph ^ k_swz<D>(r)));
    v_voff = (uint32_t)(key_of_slot(grp, r) * D + 16 * (ph ^ v_swz<D>(r)));
  }
  // The tile loads are untracked by the compiler (which would otherwise wait
  // for them before the next LDS read of any buffer); every fenced barrier
  // below waits for them explicitly.
  // position u of the walk (LDS buffer) is key tile ti (keys ti * BC ..)
  auto dma_k = [&](int u, int ti) __attribute__((always_inline)) {
    const int j0 = ti * BC;
    const uint32_t rest = (uint32_t)max(s_k - j0, 0) * D;
    if (wg < N_DMA)
      load16_to_lds_untracked(kg + (int64_t)j0 * D, rest,
                              lds + ((boff + u) & (NBUF - 1)) * BUF_BYTES + (grp * H_SLOTS + 64 * wg) * 16, k_voff);
  };
  auto dma_v = [&](int u, int ti) __attribute__((always_inline)) {
    const int j0 = ti * BC;
    const uint32_t rest = (uint32_t)max(s_k - j0, 0) * D;
    if (wg < N_DMA)
      load16_to_lds_untracked(vg + (int64_t)j0 * D, rest,
                              lds + ((boff + u) & (NBUF - 1)) * BUF_BYTES + K_BYTES + (grp * H_SLOTS + 64 * wg) * 16, v_voff);
  };

  // ---- per-wave running state
  f32x16_t o[DB];
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t sc[KB];
  float xw[KB][16];        // float32 weights of the tile between its two steps
  i32x8_t pf;              // the same rounded to E4M3 (value product operand)
  uint32_t mbyte = 1u;
  // Two ways to walk an item, as in the bf16 kernel (each an instantiation of
  // the tile walk): range (the visible keys are exactly [key_lo, key_hi); position u
  // is key tile toff + u; hidden keys by scalar arithmetic, no mask reads) and
  // list (any other mask: position u is entry u of the tile list, or key
  // tile u past the list's length; a four-entry tile ring in one vector
  // register; each tile's mask bytes are read).
  int toff = 0, key_lo = 0, key_hi = 0;
  bool use_list = false, list_identity = false;
  int ringv = 0;
  auto ring_load = [&](int t0) -> int {
    const int u = t0 + (lane & 3);
    return list_identity ? u : (int)lds_tl[min(u, kTileListMax + 7)];
  };
  // key tile at walk position t + k (k = 0 .. 3) while position t is the next V step's
  auto tile_at = [&](int t, int k, auto list) __attribute__((always_inline)) -> int {
    if constexpr (decltype(list)::value) return __builtin_amdgcn_readlane(ringv, k);
    else return toff + t + k;
  };

  // Score-product fragment reads: lane (ln, hl) reads K row 32 kb + ln at
  // logical slot 4 kk + 2 hl + u (features 64 kk + 32 hl + 16 u ..); the
  // swizzle depends on ln only (adding 32 rows leaves it unchanged).
  int k_off[DK][2];
#pragma unroll
  for (int kk = 0; kk < DK; ++kk)
#pragma unroll
    for (int u = 0; u < 2; ++u) k_off[kk][u] = ln * D + 16 * ((4 * kk + 2 * hl + u) ^ k_swz<D>(ln));
  // Transpose-read addresses of the value product's A operand. Lane L (group
  // G = L / 16, x = L % 16, half h = G / 2) reads, for byte block tb and
  // feature block db, LDS row 32 h + 8 tb + x / 2 (key key(h, 8 tb + x / 2))
  // at features 32 db + 16 (G & 1) + 8 (x & 1) .. +7; the transpose hands
  // lane L the bytes of its own feature 32 db + L % 32 for the keys of slots
  // 8 tb .. 8 tb + 7 of its half. The row's swizzle does not depend on tb,
  // and it keeps the slot's low bit, so the slot is 2 (db ^ s) + (G & 1).
  int v_off[DB];
  {
    const int row = 32 * (lane >> 5) + ((lane & 15) >> 1);
    const int sw = v_swz<D>(row) >> 1;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v_off[db] = row * D + 16 * (2 * (db ^ sw) + ((lane >> 4) & 1)) + 8 * (lane & 1);
  }
  auto v_read = [&](int t, int i) __attribute__((always_inline)) -> i32x2_t {
    // read i of tile t's value product: feature block i / 4, byte block i % 4
    const char* vl = lds + ((boff + t) & (NBUF - 1)) * BUF_BYTES + K_BYTES;
    const int db = i >> 2, tb = i & 3;
    return lds_read_tr8(vl + v_off[db] + 8 * tb * D);
  };

  constexpr int N_VR = 4 * DB;  // transpose reads per value product
  constexpr int LA = 8;         // of them issued before the M step's barrier
  static_assert(LA <= N_VR, "prefetched reads must belong to the value product");
  i32x2_t vpre[LA];
  // Operands of the two products: the value product's transpose reads (the
  // first LA of them were issued before the M step's barrier) and the score
  // product's K fragments.
  i32x2_t vr[N_VR];
  i32x8_t ka[KB][DK];
  auto read_v = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < N_VR; ++i) vr[i] = i < LA ? vpre[i < LA ? i : 0] : v_read(t, i);
  };
  auto read_k = [&](int t) __attribute__((always_inline)) {
    const char* kl = lds + ((boff + t) & (NBUF - 1)) * BUF_BYTES;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int kk = 0; kk < DK; ++kk)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4_t x = *(const u32x4_t*)(kl + k_off[kk][u] + kb * 32 * D);
#pragma unroll
          for (int e = 0; e < 4; ++e) ka[kb][kk][4 * u + e] = (int)x[e];
        }
  };
  // O^T += V_t^T P(t)^T.
  auto pv_mfma = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      i32x8_t a;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        a[2 * tb] = vr[4 * db + tb][0];
        a[2 * tb + 1] = vr[4 * db + tb][1];
      }
      o[db] = mfma_e4m3(a, pf, o[db]);
    }
  };
  // S(t)^T = K_t Q^T (the key blocks' chains interleaved).
  auto qk_mfma = [&](int t, auto list) __attribute__((always_inline)) {
    f32x16_t acc[KB];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc[kb] = mfma_e4m3(ka[kb][kk], qf[kk], kk ? acc[kb] : f32x16_t{});
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sc[kb] = acc[kb];
    if constexpr (PADMASK && decltype(list)::value) {
      const int key = tile_at(t, 0, list) * BC + lane;
      mbyte = key < s_k ? (uint32_t)mg[key] : 1u;
    }
  };
  auto qk = [&](int t, auto list) __attribute__((always_inline)) {
    read_k(t);
    qk_mfma(t, list);
  };
  // Weights of the scores in sc against the current reference max.
  auto weights = [&](float nmc) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) xw[kb][r] = fmaf(sc[kb][r], c, nmc);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) xw[kb][r] = __builtin_amdgcn_exp2f(xw[kb][r]);
  };
  auto row_sum = [&]() __attribute__((always_inline)) -> float {
    // four chains started from the first four weights (0 + w would cost an
    // add: the compiler may not fold it)
    float ps[4] = {xw[0][0], xw[0][1], xw[0][2], xw[0][3]};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb > 0 || r >= 4) ps[r & 3] += xw[kb][r];
    return (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };
  // Start of an M step: the rest of the softmax of the tile whose scores are
  // in sc (the V step before it took the exponentials). The tile's float32
  // row sum bounds every weight; if it exceeds the limit (or overflowed) in
  // any lane, the wave takes the true max, rescales O and l by
  // exp2((m_old - m_new) c) and recomputes the weights (a lane whose row has
  // no visible key yet keeps alpha = 1). Then the weights are rounded to E4M3
  // as the value product's operand. This vector work sits in the M step
  // because the V step, with the exponentials, is the longer of the two.
  auto finish = [&]() __attribute__((always_inline)) {
    float rs = row_sum();
    if (__ballot(!(rs <= kSumLimit)) != 0ull) {
      float mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const bool none = m_new == -INFINITY;
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      weights(none ? 0.f : -m_new * c);
      rs = row_sum();
    }
    l_run += rs;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, r0 = 4 * (w & 3);
      pf[w] = (int)pack_e4m3(xw[kb][r0], xw[kb][r0 + 1], xw[kb][r0 + 2], xw[kb][r0 + 3]);
    }
  };
  // One M step: every LDS read first, then the softmax tail (its vector work
  // covers the read latency), then the eight MFMAs.
  auto m_step = [&](int tp, int tq, auto list) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(2);
    read_v(tp);
    read_k(tq);
    finish();
    pv_mfma();
    qk_mfma(tq, list);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  };
  // V step: staging of later tiles, then masks and the exponentials of S(t).
  auto vstep = [&](int t, auto list) __attribute__((always_inline)) {
    constexpr bool LIST = decltype(list)::value;
    // the next four list entries, read before this step's loads
    int ring_new = 0;
    if constexpr (LIST) ring_new = ring_load(t + 1);
    dma_k(t + 3, tile_at(t, 3, list));
    dma_v(t + 2, tile_at(t, 2, list));
    const int j0 = tile_at(t, 0, list) * BC;
    uint64_t hid;
    if constexpr (PADMASK && LIST) {
      hid = __ballot(mbyte != 0u);
    } else {
      hid = hidden_outside(j0, key_lo, key_hi);
    }
    if (hid != 0ull || (CAUSAL && j0 + BC - 1 > qlo)) {
      // register r of block kb holds key offset 32 kb + 8 (r / 4) + 4 hl + r % 4
      const uint64_t hsh = hid >> (4 * hl);
      const int lim = qlo + ln - j0 - 4 * hl;  // causal: visible iff offset - 4 hl <= lim
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t w = (uint32_t)(hsh >> (32 * kb));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 8 * (r >> 2) + (r & 3);
          const bool hide = ((w >> kr) & 1u) || (CAUSAL && 32 * kb + kr > lim);
          if (hide) sc[kb][r] = -INFINITY;
        }
      }
    }
    // (walking a range, every row that sees any key sees key key_lo, in tile 0)
    if ((PADMASK && LIST) ? (__ballot(m_run == -INFINITY) != 0ull) : (t == 0)) {
      float mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (m_run == -INFINITY) m_run = mx;
    }
    weights(-((m_run == -INFINITY) ? 0.f : m_run) * c);
    if constexpr (LIST) ringv = ring_new;
  };

  // ---- the workgroup's items, one after the other
  for (;;) {
    const int L = L_cur;
    const int L_next = item_of(round + 1);
    const bool has_next = PERSIST && L_next < p.n_items;
    const int qt = CAUSAL ? (p.n_qt - 1 - L / p.BH) : (L / p.BH);
    bh = L % p.BH;
    b = bh / p.H;
    q0 = qt * BR;
    // Per-head score scale: scores enter exp2 as (q8 . k8) * c with
    // c = |scale * dq * dk| * log2(e); a negative product negates Q (the sign
    // bit of each code), a zero one zeroes Q.
    const float dq = p.dsq ? p.dsq[bh] : 1.f;
    const float dk = p.dsk ? p.dsk[bh] : 1.f;
    dv = p.dsv ? p.dsv[bh] : 1.f;
    const float cs = p.scale * dq * dk;
    const float cs_abs = fabsf(cs);
    const bool zero_scale = cs_abs < 1e-30f;  // NaN propagates
    q_and = zero_scale ? 0u : ~0u;
    q_xor = (!zero_scale && cs < 0.f) ? 0x80808080u : 0u;
    c = zero_scale ? kLog2e : cs_abs * kLog2e;
    scale_abs = zero_scale ? 0.f : cs_abs;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (int64_t)bh * s_q * D, (uint32_t)s_q * D);
    kg = p.k + (int64_t)bh * s_k * D;
    vg = p.v + (int64_t)bh * s_k * D;
    mg = PADMASK ? p.kpm + (int64_t)b * s_k : nullptr;

    // ---- keys this tile can see: causal stops at the last query row; with a
    // padding mask only the tiles that hold a visible key are walked
    int kend = s_k;
    if (CAUSAL) kend = min(kend, q0 + BR);
    const int n_t = kend > 0 ? (kend + BC - 1) / BC : 0;
    toff = 0;
    key_lo = 0;
    key_hi = s_k;
    use_list = false;
    list_identity = false;
    if (PADMASK && n_t <= kTileListMax) {
      int contig = 1;
      n_kv = build_tile_list<BC, NT / 64>(mg, kend, n_t, lds_bits, lds_tl, lds_scr, &key_lo, &key_hi, &contig);
      use_list = contig == 0;
      if (!use_list) {  // visible keys [key_lo, key_hi): walk their tiles as a range
        toff = key_lo / BC;
        n_kv = key_hi > key_lo ? (key_hi - 1) / BC - toff + 1 : 0;
      }
    } else if (PADMASK) {
      // a long item: walk every tile up to the last key that is not padded
      if (tid == 0) lds_last = -1;
      __syncthreads();
      int last = -1;
      for (int cend = s_k; cend > 0; cend -= NT * 4) {
        const int cbeg = max(0, cend - NT * 4);
        int best = -1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = cbeg + tid * 4 + i;
          if (j < cend && mg[j] == 0) best = j;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) best = max(best, __shfl_xor(best, off));
        if (lane == 0 && best >= 0) atomicMax(&lds_last, best);
        __syncthreads();
        const int found = lds_last;
        __syncthreads();
        if (found >= 0) {
          last = found;
          break;
        }
      }
      kend = min(kend, last + 1);
      n_kv = kend > 0 ? (kend + BC - 1) / BC : 0;
      use_list = true;
      list_identity = true;
    } else {
      n_kv = n_t;
    }

    // ---- Q (B operand of the score product): lane holds query qlo + ln,
    // features 64 kk + 32 hl .. +31
    qlo = q0 + 32 * wv;
    {
      const uint32_t row = (uint32_t)(qlo + ln);
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4_t x = load16(rq, row * D + 64 * kk + 32 * hl + 16 * u);
          x = (x & q_and) ^ q_xor;
#pragma unroll
          for (int e = 0; e < 4; ++e) qf[kk][4 * u + e] = (int)x[e];
        }
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};
    m_run = -INFINITY;
    l_run = 0.f;
    mbyte = 1u;

    // the first tiles' loads (positions 0 .. 2); selects rather than a branch
    // on the kind of walk (a branch here made the compiler spill)
    if (PADMASK) ringv = ring_load(0);
    auto first_tile = [&](int k) -> int {
      return (PADMASK && use_list) ? __builtin_amdgcn_readlane(ringv, k) : toff + k;
    };
    if (n_kv > 0) {
      dma_k(0, first_tile(0));
      dma_k(1, first_tile(1));
      dma_k(2, first_tile(2));
      dma_v(0, first_tile(0));
      dma_v(1, first_tile(1));
    }
    wait_loads();
    __syncthreads();

    // ---- ping-pong schedule, as in the bf16 kernel: n_kv + 2 intervals, each
    // closed by a workgroup barrier. Interval 0: group 0 runs QK(0). Interval
    // t + 1 (t < n_kv): group 0 runs V(t) then M(t + 1), group 1 M(t) then V(t)
    // (M(n_kv) is PV(n_kv - 1) alone). Interval n_kv + 1: group 1 runs
    // PV(n_kv - 1). LDS buffer u % 4 holds tile u. K(u) is requested by V(u - 3)
    // in interval u - 2 and read by QK(u) in intervals u (group 0) and u + 1
    // (group 1); V(u) is requested by V(u - 2) in interval u - 1 and read from
    // the prefetch at the end of V(u) (interval u + 1) to PV(u) of group 1
    // (interval u + 2). Every request comes after the last read of tile u - 4
    // (K: interval u - 3, V: interval u - 2) and is waited for (explicitly: the
    // requests are untracked) at the barrier closing its interval.
    auto phase_sync = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      wait_loads();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    // End of V(t): the first LA reads of PV(t) are issued here, so their
    // latency overlaps the switch to the M step.
    auto vstep_end = [&](int t) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < LA; ++i) vpre[i] = v_read(t, i);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto walk = [&](auto list) __attribute__((always_inline)) {
      if (grp == 0) {
        qk(0, list);
        phase_sync();
        for (int t = 0; t < n_kv - 1; ++t) {
          vstep(t, list);
          vstep_end(t);
          m_step(t, t + 1, list);
          phase_sync();
        }
        vstep(n_kv - 1, list);
        vstep_end(n_kv - 1);
        read_v(n_kv - 1);
        finish();
        pv_mfma();
        phase_sync();
        phase_sync();
      } else {
        phase_sync();
        qk(0, list);
        vstep(0, list);
        vstep_end(0);
        phase_sync();
        for (int t = 1; t < n_kv; ++t) {
          m_step(t - 1, t, list);
          vstep(t, list);
          vstep_end(t);
          phase_sync();
        }
        read_v(n_kv - 1);
        finish();
        pv_mfma();
        phase_sync();
      }
    };
    if (n_kv > 0) {
      if (PADMASK && use_list)
        walk(std::true_type{});
      else
        walk(std::false_type{});
    }

    // ---- epilogue: O = dv * O^T / l, lse = m |scale dq dk| + ln(l)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? dv * __builtin_amdgcn_rcpf(l_tot) : 0.f;
    const int row = qlo + ln;
    if (row < s_q) {
      uint16_t* og = p.out + ((int64_t)bh * s_q + row) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2_t w;
          w[0] = pack_bf16(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
          w[1] = pack_bf16(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
          *(u32x2_t*)(og + 32 * db + 8 * g + 4 * hl) = w;
        }
      }
      if (hl == 0) {
        p.lse[(int64_t)bh * s_q + row] =
            l_tot > 0.f ? m_run * scale_abs + __builtin_amdgcn_logf(l_tot) * kLn2 : -INFINITY;
      }
    }
    if (!has_next) break;
    boff = (boff + n_kv) & (NBUF - 1);
    L_cur = L_next;
    ++round;
  }
}

template <int D, bool CAUSAL, bool PADMASK>
hipError_t launch(const Fp8Params& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, CAUSAL, PADMASK>), dim3(grid), dim3(512), 0, stream, p);
  return hipGetLastError();
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

}  // namespace

extern "C" int attn_fwd_fp8_validate(const void* q, const void* k, const void* v,
                                     const float* descale_q, const float* descale_k,
                                     const float* descale_v, const void* out, const float* lse,
                                     int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d,
                                     float scale, int causal, const uint8_t* key_padding_mask) {
  (void)causal;
  if (B < 0 || H < 0 || s_q < 0 || s_k < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  const int64_t kMaxSeq = (int64_t)1 << 22;
  if (s_q > kMaxSeq || s_k > kMaxSeq) return ATTN_ERR_SHAPE;
  if (H > 0 && B > INT32_MAX / H) return ATTN_ERR_SHAPE;
  const int64_t BH = B * H;
  // the work items (B * H * query tiles) must fit a 32-bit int
  if (BH * ((s_q + 255) / 256) > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  if (BH == 0 || s_q == 0) return ATTN_OK;
  if (!q || !out || !lse) return ATTN_ERR_NULL;
  if (s_k > 0 && (!k || !v)) return ATTN_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)out) & 15u) return ATTN_ERR_ALIGN;
  if (s_k > 0 && (((uintptr_t)k | (uintptr_t)v) & 15u)) return ATTN_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)descale_q | (uintptr_t)descale_k | (uintptr_t)descale_v) & 3u)
    return ATTN_ERR_ALIGN;
  const int64_t nq = BH * s_q * d, nk = BH * s_k * d, no = BH * s_q * d * 2, nl = BH * s_q * 4;
  const int64_t nm = key_padding_mask ? B * s_k : 0, nd = BH * 4;
  const void* ins[7] = {q, k, v, key_padding_mask, descale_q, descale_k, descale_v};
  const int64_t ns[7] = {nq, nk, nk, nm, nd, nd, nd};
  for (int i = 0; i < 7; ++i) {
    if (overlaps(out, no, ins[i], ns[i]) || overlaps(lse, nl, ins[i], ns[i])) return ATTN_ERR_ALIAS;
  }
  if (overlaps(out, no, lse, nl)) return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

extern "C" int attn_fwd_fp8(const void* q, const void* k, const void* v, const float* descale_q,
                            const float* descale_k, const float* descale_v, void* out, float* lse,
                            int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d, float scale,
                            int causal, const uint8_t* key_padding_mask, void* stream) {
  const int st = attn_fwd_fp8_validate(q, k, v, descale_q, descale_k, descale_v, out, lse, B, H,
                                       s_q, s_k, d, scale, causal, key_padding_mask);
  if (st != ATTN_OK) return st;
  if (B * H == 0 || s_q == 0) return ATTN_OK;
  Fp8Params p = {};
  p.q = (const uint8_t*)q;
  p.k = (const uint8_t*)k;
  p.v = (const uint8_t*)v;
  p.dsq = descale_q;
  p.dsk = descale_k;
  p.dsv = descale_v;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.kpm = key_padding_mask;
  p.s_q = (int)s_q;
  p.s_k = (int)s_k;
  p.H = (int)H;
  p.BH = (int)(B * H);
  p.n_qt = (int)((s_q + 255) / 256);
  p.scale = scale;
  p.n_items = p.BH * p.n_qt;
  const bool pad = key_padding_mask != nullptr && s_k > 0;
  const bool cz = causal != 0;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e;
  // one workgroup per item at d = 128, a persistent grid at d = 64
  int grid = p.n_items;
  if (d == 64) {
    int n_cu = 0;
    e = cu_count(&n_cu);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return ATTN_ERR_LAUNCH;
    }
    if (grid > n_cu) grid = n_cu;
  }
  if (d == 128) {
    e = cz ? (pad ? launch<128, true, true>(p, grid, hs) : launch<128, true, false>(p, grid, hs))
           : (pad ? launch<128, false, true>(p, grid, hs) : launch<128, false, false>(p, grid, hs));
  } else {
    e = cz ? (pad ? launch<64, true, true>(p, grid, hs) : launch<64, true, false>(p, grid, hs))
           : (pad ? launch<64, false, true>(p, grid, hs) : launch<64, false, false>(p, grid, hs));
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_LAUNCH;
  }
  g_last_hip_error = 0;
  return ATTN_OK;
}
