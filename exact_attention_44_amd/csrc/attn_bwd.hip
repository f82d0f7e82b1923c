// attn_bwd.hip - attention backward pass for gfx950 (CDNA4) and its C ABI.
//
// Gradients of O = softmax(scale Q K^T + mask) V for a given dO. The onecalc.app
// page "Attention memory" (section "What this memory is") notes that a training
// framework keeps the materialised score matrix for the backward pass unless a
// fused kernel does without it; here nothing of size s_q x s_k is stored: the
// weights are rebuilt tile by tile from the forward pass's log-sum-exp,
// P = exp(scale q.k - lse), as in the forward's block-wise walk (news.hamidun.com
// glossary "Flash attention", second paragraph). The chain rule through the
// definition's steps gives, per row i,
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij = dO_i . O_i,
//   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels, launched in order on one stream:
//   dq kernel   one workgroup per (b, h, 128-query tile), 4 waves of 32 query
//               rows; walks the key tiles: S^T = K Q^T and dP^T = V dO^T
//               (the query side stays in registers, one query per lane, as in
//               the forward), dS, then dQ^T += K^T dS^T. It also writes D.
//   dkv kernel  one workgroup per (b, h, 128-key tile), 4 waves of 32 keys;
//               walks the query tiles: S = Q K^T and dP = dO V^T (the key side
//               stays in registers, one key per lane), dS, then
//               dV^T += dO^T P and dK^T += Q^T dS. At d = 128 its wave-pair
//               form runs instead: 8 waves, the two of a SIMD sharing 32 keys,
//               one computing S, P and dV, the other dP, dS and dK.
// In both, the rows of the LDS operand are read in the permuted order of
// key_of_row, so the 32x32 accumulators are the bf16 operands of the next
// product after a conversion, with no shuffles. The tiles that walk (K and V
// in the dq kernel, Q and dO in the dkv kernel) are loaded straight into LDS,
// row-major, and the transposed operands of the gradient products are read
// with LDS transpose reads. The dkv kernel also loads the rows' lse*log2(e)
// and D, which the dq kernel writes to the workspace.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "attn.h"
#include "attn_common.h"

namespace {

using namespace attn_detail;

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;        // D = rowsum(dO * O), float32 [B*H][s_qp] (workspace)
  float* lse2w;        // lse * log2(e), -inf for empty or padding rows, [B*H][s_qp]
  const uint8_t* kpm;
  int s_q, s_k, H, BH, n_qt, n_kt;
  int s_qp;            // s_q rounded up to 128: workspace rows per (b, h)
  float c;             // scale * log2(e): weights are exp2(q.k c - lse log2(e))
  float scale;
};

// Last unpadded key + 1 of batch item b (0 if all are padded); every thread
// of the workgroup gets the value.
__device__ int keys_until_last_unpadded(const uint8_t* mg, int s_k, int* lds_last) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63;
  if (tid == 0) *lds_last = -1;
  __syncthreads();
  int last = -1;
  for (int cend = s_k; cend > 0; cend -= nt * 4) {
    const int cbeg = max(0, cend - nt * 4);
    int best = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = cbeg + tid * 4 + i;
      if (j < cend && mg[j] == 0) best = j;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) best = max(best, __shfl_xor(best, off));
    if (lane == 0 && best >= 0) atomicMax(lds_last, best);
    __syncthreads();
    const int found = *lds_last;
    __syncthreads();
    if (found >= 0) {
      last = found;
      break;
    }
  }
  return last + 1;
}

// ---------------------------------------------------------------------------
// dq kernel
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool PADMASK>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdParams p) {
  // 32-key tiles at d = 128 keep the kernel within 256 registers, so two
  // workgroups share a CU and one's staging and softmax overlap the other's
  // matrix work
  constexpr int NT = 256, BR = 128, BC = D == 128 ? 32 : 64;
  constexpr int KB = BC / 32, DK = D / 16, DB = D / 32;
  constexpr int RB = 2 * D;               // bytes per K / V row in LDS
  constexpr int SL = D / 8;               // 16-byte slots per row
  constexpr int TILE = BC * RB;           // one K or V tile
  constexpr int BUF = 2 * TILE;
  constexpr int NQ = BC * SL / NT;        // loads per wave per K or V tile
  static_assert((BC * SL) % NT == 0, "a tile is a whole number of loads per wave");

  __shared__ __attribute__((aligned(16))) char lds[2 * BUF];
  __shared__ int lds_last;
  // With a padding mask: the key tiles that hold a visible key, in order (see
  // build_tile_list); a longer key range walks every tile up to the last
  // unpadded key.
  __shared__ uint16_t lds_tl[PADMASK ? kTileListMax + 8 : 1];
  __shared__ __attribute__((aligned(8))) uint8_t lds_bits[PADMASK ? kTileListMax / 8 : 8];
  __shared__ int lds_scr[3 * (NT / 64) + 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ln = lane & 31;
  const int L = blockIdx.x;
  const int qt = CAUSAL ? (p.n_qt - 1 - L / p.BH) : (L / p.BH);
  const int bh = L % p.BH, b = bh / p.H;
  const int q0 = qt * BR;
  const int s_q = p.s_q, s_k = p.s_k;
  const uint16_t* kg = p.k + (int64_t)bh * s_k * D;
  const uint16_t* vg = p.v + (int64_t)bh * s_k * D;
  const uint8_t* mg = PADMASK ? p.kpm + (int64_t)b * s_k : nullptr;

  int kend = s_k;
  if (CAUSAL) kend = min(kend, q0 + BR);
  const int n_t = kend > 0 ? (kend + BC - 1) / BC : 0;
  int n_kv = n_t;
  // walk position u is key tile toff + u, or entry u of the tile list when
  // the visible tiles are not contiguous
  int toff = 0, contig = 1;
  if (PADMASK && n_t <= kTileListMax) {
    int ka = 0, kb = 0;
    n_kv = build_tile_list<BC, NT / 64>(mg, kend, n_t, lds_bits, lds_tl, lds_scr, &ka, &kb, &contig);
    if (contig) {  // visible keys [ka, kb): their tiles as a range
      toff = ka / BC;
      n_kv = kb > ka ? (kb - 1) / BC - toff + 1 : 0;
    }
  } else if (PADMASK) {
    kend = min(kend, keys_until_last_unpadded(mg, s_k, &lds_last));
    n_kv = kend > 0 ? (kend + BC - 1) / BC : 0;
  }
  const bool use_list = PADMASK && contig == 0;
  // Key tiles at walk positions t .. t + 3 in lanes 0 .. 3 of one register
  // (t: the current iteration).
  auto ring_load = [&](int t0) -> int {
    const int u = t0 + (lane & 3);
    return use_list ? (int)lds_tl[min(u, kTileListMax + 7)] : toff + u;
  };
  int ringv = PADMASK ? ring_load(0) : 0;
  auto ring_at = [&](int k) -> int { return __builtin_amdgcn_readlane(ringv, k); };

  // query side, one query per lane: Q and dO fragments (B operands), O for D
  const int qlo = q0 + 32 * wv;
  const int row = qlo + ln;
  bf16x8_t qf[DK], df[DK];
  float dsum = 0.f;
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (int64_t)bh * s_q * D, (uint32_t)s_q * D * 2);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dout + (int64_t)bh * s_q * D, (uint32_t)s_q * D * 2);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o + (int64_t)bh * s_q * D, (uint32_t)s_q * D * 2);
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
      const uint32_t off = (uint32_t)(row * D + 16 * kk + 8 * hl) * 2;
      qf[kk] = __builtin_bit_cast(bf16x8_t, load16(rq, off));
      df[kk] = __builtin_bit_cast(bf16x8_t, load16(rd, off));
      const bf16x8_t of = __builtin_bit_cast(bf16x8_t, load16(ro, off));
#pragma unroll
      for (int e = 0; e < 8; ++e) dsum = fmaf((float)df[kk][e], (float)of[e], dsum);
    }
  }
  const float Dv = dsum + __shfl_xor(dsum, 32);
  const float lse_row = row < s_q ? p.lse[(int64_t)bh * s_q + row] : -INFINITY;
  const bool live = lse_row != -INFINITY;  // a row with no visible key has P = 0
  const bool any_dead = __ballot(!live) != 0ull;
  const float lse2 = live ? lse_row * kLog2e : 0.f;
  // D and lse*log2(e) for the dkv kernel, which loads them 128 rows at a time:
  // the rows up to the next multiple of 128 are written too (D = 0, lse = -inf,
  // so they carry no weight)
  if (hl == 0 && row < p.s_qp) {
    const int64_t wi = (int64_t)bh * p.s_qp + row;
    p.delta[wi] = row < s_q ? Dv : 0.f;
    p.lse2w[wi] = (row < s_q && live) ? lse2 : -INFINITY;
  }

  // Staging: loads that write LDS directly (as in the dkv kernel). Load i of
  // this wave fills LDS slots 64 (4 i + wv) .. +63 of the K and of the V tile.
  // Keys past s_k read zeros.
  uint32_t k_voff[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int sl = 64 * (4 * i + wv) + lane;
    const int r = sl / SL, ph = sl % SL;
    k_voff[i] = (uint32_t)(r * RB + 16 * (ph ^ q_swz<D>(r)));
  }
  // key tile ti into LDS buffer bi
  auto dma_tile = [&](int ti, int bi) {
    const int j0 = ti * BC;
    char* base = lds + bi * BUF;
    const uint32_t rest = (uint32_t)max(s_k - j0, 0) * RB;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + (int64_t)j0 * D, rest);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + (int64_t)j0 * D, rest);
#pragma unroll
    for (int i = 0; i < NQ; ++i) load16_to_lds(rk, base + 64 * (4 * i + wv) * 16, k_voff[i]);
#pragma unroll
    for (int i = 0; i < NQ; ++i) load16_to_lds(rv, base + TILE + 64 * (4 * i + wv) * 16, k_voff[i]);
  };

  f32x16_t dqt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqt[db] = f32x16_t{};
  // score-side fragment offsets (row key_of_row(ln) of each 32-row block,
  // logical slot 2 kk + hl) and transpose-read offsets of K^T (see the dkv
  // kernel, which reads its Q^T and dO^T the same way)
  int a_off[DK];
  {
    const int r = key_of_row(ln);
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) a_off[kk] = r * RB + 16 * ((2 * kk + hl) ^ q_swz<D>(r));
  }
  int t_off[2][DB];
  {
    const int a = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int rw = 8 * hl + 4 * r + (a >> 2);
        const int slot = 4 * db + 2 * g + ((a & 3) >> 1);
        t_off[r][db] = rw * RB + 16 * (slot ^ q_swz<D>(rw)) + 8 * (a & 1);
      }
  }

  if (n_kv > 0) dma_tile(PADMASK ? ring_at(0) : 0, 0);
  uint32_t mbyte = 1u;  // this lane's padding byte of the current tile
  __syncthreads();
  for (int t = 0; t < n_kv; ++t) {
    // the next iteration's list entries, read before this iteration's loads
    const int ring_new = PADMASK ? ring_load(t + 1) : 0;
    const int j0 = (PADMASK ? ring_at(0) : t) * BC;
    // the padding byte before the tile loads: the vote below then waits for
    // the byte alone, not for the loads issued after it
    if (PADMASK) {
      mbyte = mg[min(j0 + lane, s_k - 1)];
      __builtin_amdgcn_sched_barrier(0);
    }
    // the other buffer was last read in the previous iteration, before its
    // closing barrier; this barrier's wait also covers the new loads
    if (t + 1 < n_kv) dma_tile(PADMASK ? ring_at(1) : t + 1, (t + 1) & 1);
    const char* kl = lds + (t & 1) * BUF;
    const char* vl = kl + TILE;
    // S^T = K Q^T and dP^T = V dO^T, one 32-key block at a time
    f32x16_t sc[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16_t a1 = {}, a2 = {};
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) {
        const bf16x8_t fk = *(const bf16x8_t*)(kl + a_off[kk] + kb * 32 * RB);
        const bf16x8_t fv = *(const bf16x8_t*)(vl + a_off[kk] + kb * 32 * RB);
        a1 = mfma(fk, qf[kk], a1);
        a2 = mfma(fv, df[kk], a2);
      }
      sc[kb] = a1;
      dp[kb] = a2;
    }
    // masks: keys past s_k or padded, and causal (key j hidden from row i when j > i)
    uint64_t hid;
    if (PADMASK) {
      // the byte was requested before the score products, from a clamped
      // address (a load under a branch would be waited for at once); keys
      // past s_k are hidden here. Lanes past BC vote on keys of the next
      // tile; their bits are unused.
      hid = __ballot(j0 + lane >= s_k || mbyte != 0u);
    } else {
      const int rem = s_k - j0;
      hid = rem >= BC ? 0ull : ~((1ull << rem) - 1ull);
    }
    const int lim = row - j0;  // causal: key offset visible iff <= lim
    // per-element masks only where the tile needs them (wave-uniform test):
    // hidden keys, the causal diagonal, or a row with no visible key
    const bool masked = hid != 0ull || (CAUSAL && j0 + BC - 1 > qlo) || any_dead;
    bf16x8_t pf[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t sh = (uint32_t)(hid >> (32 * kb)) >> (8 * hl);
      float ds[16];
      if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = 32 * kb + 16 * (r >> 3) + 8 * hl + (r & 7);
          const bool hide = !live | (((sh >> (16 * (r >> 3) + (r & 7))) & 1u) != 0u) | (CAUSAL && ko > lim);
          const float pw = __builtin_amdgcn_exp2f(hide ? -INFINITY : fmaf(sc[kb][r], p.c, -lse2));
          ds[r] = pw * (dp[kb][r] - Dv);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ds[r] = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], p.c, -lse2)) * (dp[kb][r] - Dv);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) w[e2] = pack_bf16(ds[8 * ks + 2 * e2], ds[8 * ks + 2 * e2 + 1]);
        pf[kb][ks] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    // dQ^T += K^T dS^T (A: transpose reads of the key tile)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2_t k0v = lds_read_tr16(kl + t_off[0][db] + (32 * kb + 16 * ks) * RB);
          const u32x2_t k1v = lds_read_tr16(kl + t_off[1][db] + (32 * kb + 16 * ks) * RB);
          const u32x4_t a = {k0v[0], k0v[1], k1v[0], k1v[1]};
          dqt[db] = mfma(__builtin_bit_cast(bf16x8_t, a), pf[kb][ks], dqt[db]);
        }
    __syncthreads();
    if (PADMASK) ringv = ring_new;
  }

  if (row < s_q) {
    uint16_t* g = p.dq + ((int64_t)bh * s_q + row) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        u32x2_t w;
        w[0] = pack_bf16(dqt[db][4 * gi + 0] * p.scale, dqt[db][4 * gi + 1] * p.scale);
        w[1] = pack_bf16(dqt[db][4 * gi + 2] * p.scale, dqt[db][4 * gi + 3] * p.scale);
        *(u32x2_t*)(g + 32 * db + 8 * gi + 4 * hl) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dkv kernel
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool PADMASK>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void attn_bwd_dkv_kernel(BwdParams p) {
  constexpr int NT = 256, BK = 128, BQ = 128;
  constexpr int QB = BQ / 32, DK = D / 16, DB = D / 32;
  constexpr int RB = 2 * D;                   // bytes per Q / dO row in LDS
  constexpr int SL = D / 8;                   // 16-byte slots per row
  constexpr int TILE = BQ * RB;               // one Q or dO tile
  constexpr int BUF = 2 * TILE + 2 * BQ * 4;  // Q, dO, lse*log2e, D
  constexpr int NQ = BQ * SL / NT;            // loads per wave per Q or dO tile
  static_assert((BQ * SL) % NT == 0, "a tile is a whole number of loads per wave");

  __shared__ __attribute__((aligned(16))) char lds[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ln = lane & 31;
  const int L = blockIdx.x;
  const int kt = L / p.BH;
  const int bh = L % p.BH, b = bh / p.H;
  const int k0 = kt * BK;
  const int s_q = p.s_q, s_k = p.s_k;

  // key side, one key per lane: K and V fragments (B operands)
  const int key = k0 + 32 * wv + ln;
  bf16x8_t kf[DK], vf[DK];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (int64_t)bh * s_k * D, (uint32_t)s_k * D * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (int64_t)bh * s_k * D, (uint32_t)s_k * D * 2);
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
      const uint32_t off = (uint32_t)(key * D + 16 * kk + 8 * hl) * 2;
      kf[kk] = __builtin_bit_cast(bf16x8_t, load16(rk, off));
      vf[kk] = __builtin_bit_cast(bf16x8_t, load16(rv, off));
    }
  }
  bool kvis = key < s_k;
  if (PADMASK && kvis) kvis = p.kpm[(int64_t)b * s_k + key] == 0;
  // causal: this key is hidden from query qi when kcut > qi (every query
  // when the key itself is hidden)
  const int kcut = kvis ? key : INT_MAX;
  // Without a padding mask every row below s_q sees a key (lse > -inf); with
  // all of this wave's keys visible, only causal diagonal blocks and the
  // ragged last block need masks.
  const bool keys_masked = PADMASK || __ballot(!kvis) != 0ull;
  const int kmax = k0 + 32 * wv + 31;  // this wave's last key

  // query tiles that can see a key of this tile; none when every key of the
  // block is padded (its gradients are zero)
  const int qt0 = CAUSAL ? min(k0, s_q) / BQ : 0;
  int qt1 = (s_q + BQ - 1) / BQ;
  if (PADMASK && !__syncthreads_or(kvis)) qt1 = qt0;
  const uint16_t* qg = p.q + (int64_t)bh * s_q * D;
  const uint16_t* dg = p.dout + (int64_t)bh * s_q * D;
  const float* l2g = p.lse2w + (int64_t)bh * p.s_qp;
  const float* Dg = p.delta + (int64_t)bh * p.s_qp;

  // Staging: loads that write LDS directly. Load i of this wave fills LDS
  // slots 64 (4 i + wv) .. +63 of the Q and of the dO tile; each lane loads
  // the memory slot that belongs in its LDS slot. Rows past s_q read zeros.
  uint32_t q_voff[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int sl = 64 * (4 * i + wv) + lane;
    const int r = sl / SL, ph = sl % SL;
    q_voff[i] = (uint32_t)(r * RB + 16 * (ph ^ q_swz<D>(r)));
  }
  auto dma_tile = [&](int u, int bi) {
    const int i0 = u * BQ;
    char* base = lds + bi * BUF;
    const uint32_t rest = (uint32_t)max(s_q - i0, 0) * RB;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg + (int64_t)i0 * D, rest);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dg + (int64_t)i0 * D, rest);
#pragma unroll
    for (int i = 0; i < NQ; ++i) load16_to_lds(rq, base + 64 * (4 * i + wv) * 16, q_voff[i]);
#pragma unroll
    for (int i = 0; i < NQ; ++i) load16_to_lds(rd, base + TILE + 64 * (4 * i + wv) * 16, q_voff[i]);
    // lse*log2e then D of the tile's BQ rows, BQ / 4 slots each: wave wv
    // loads slots LS (wv & 1) .. +LS-1 of lse*log2e (waves 0, 1) or of D
    // (waves 2, 3). The workspace holds s_qp >= i0 + BQ rows per (b, h).
    constexpr int LS = BQ / 8;
    const __amdgpu_buffer_rsrc_t rl = make_rsrc((wv < 2 ? l2g : Dg) + i0, BQ * 4);
    if (lane < LS) load16_to_lds(rl, base + 2 * TILE + 16 * LS * wv, (uint32_t)(16 * (LS * (wv & 1) + lane)));
  };

  f32x16_t dkt[DB], dvt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkt[db] = f32x16_t{};
    dvt[db] = f32x16_t{};
  }
  // Score-side fragment reads: lane (ln, hl) reads row key_of_row(ln) of each
  // 32-row block at logical slot 2 kk + hl (features 16 kk + 8 hl ..).
  int a_off[DK];
  {
    const int r = key_of_row(ln);
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) a_off[kk] = r * RB + 16 * ((2 * kk + hl) ^ q_swz<D>(r));
  }
  // Transpose reads of the gradient products' A operands (Q^T, dO^T: rows =
  // features, k = 16 queries of a k-step). Lane a of 16-lane group G (half
  // hl = G / 2, g = G & 1) gives, for read r of feature block db, the address
  // of query row 8 hl + 4 r + a / 4 of the k-step at features
  // 32 db + 16 g + 4 (a & 3) .. +3; lane L then holds feature 32 db + L % 32 of
  // queries 8 hl + 4 r .. +3, elements 4 r .. 4 r + 3 of its operand.
  int t_off[2][DB];
  {
    const int a = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 8 * hl + 4 * r + (a >> 2);
        const int slot = 4 * db + 2 * g + ((a & 3) >> 1);
        t_off[r][db] = row * RB + 16 * (slot ^ q_swz<D>(row)) + 8 * (a & 1);
      }
  }
  const int n_it = qt1 - qt0;

  if (n_it > 0) dma_tile(qt0, 0);
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    const int u = qt0 + it;
    // the other buffer was last read in the previous iteration, before its
    // closing barrier; this barrier's wait also covers the new loads
    if (it + 1 < n_it) dma_tile(u + 1, (it + 1) & 1);
    const char* ql = lds + (it & 1) * BUF;
    const char* dl = ql + TILE;
    const float* lw = (const float*)(ql + 2 * TILE);
    const int i0 = u * BQ;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // Three scheduling regions per 32-query block. One wave per SIMD hides
      // LDS latency only by issuing reads ahead of their use:
      // (1) the score-side fragments, LA reads ahead of the 16 score MFMAs;
      // (2) the 32 transpose reads of the gradient operands, then the vector
      //     work (P, dS) that covers their latency;
      // (3) the 16 gradient MFMAs.
      constexpr int LA = D == 128 ? 8 : 6;
      f32x4_t lv[4], dv4[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int qo = 32 * qb + 16 * h2 + 8 * hl;
        lv[2 * h2] = *(const f32x4_t*)(lw + qo);
        lv[2 * h2 + 1] = *(const f32x4_t*)(lw + qo + 4);
        dv4[2 * h2] = *(const f32x4_t*)(lw + BQ + qo);
        dv4[2 * h2 + 1] = *(const f32x4_t*)(lw + BQ + qo + 4);
      }
      // S = Q K^T and dP = dO V^T for 32 queries: one key per lane, the
      // registers hold queries 32qb + {8h..8h+7, 16+8h..16+8h+7}
      f32x16_t s = {}, dp = {};
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) {
        const bf16x8_t fq = *(const bf16x8_t*)(ql + a_off[kk] + qb * 32 * RB);
        const bf16x8_t fd = *(const bf16x8_t*)(dl + a_off[kk] + qb * 32 * RB);
        s = mfma(fq, kf[kk], s);
        dp = mfma(fd, vf[kk], dp);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8 + LA, 0);
#pragma unroll
      for (int i = 0; i < 2 * DK - LA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
      __builtin_amdgcn_sched_barrier(0);
      u32x2_t tq[2][DB][2], td[2][DB][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int o = t_off[r][db] + (32 * qb + 16 * ks) * RB;
            td[ks][db][r] = lds_read_tr16(dl + o);
            tq[ks][db][r] = lds_read_tr16(ql + o);
          }
      float lr[16], dr[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lr[4 * q4 + e] = lv[q4][e];
          dr[4 * q4 + e] = dv4[q4][e];
        }
      float pw[16], ds[16];
      // masks where a key is hidden, on the causal diagonal, and on the
      // ragged last block (its rows past s_q carry lse = -inf)
      if (keys_masked || (CAUSAL && i0 + 32 * qb < kmax) || i0 + 32 * qb + 32 > s_q) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = i0 + 32 * qb + 16 * (r >> 3) + 8 * hl + (r & 7);
          // bitwise, not short-circuit, so the test stays straight-line code
          const bool hide = (lr[r] == -INFINITY) | (CAUSAL ? (kcut > qi) : !kvis);
          // a hidden weight is exp2(-inf) = 0: selecting the argument keeps the
          // exponential unconditional (a select on the result becomes a branch)
          pw[r] = __builtin_amdgcn_exp2f(hide ? -INFINITY : fmaf(s[r], p.c, -lr[r]));
          ds[r] = pw[r] * (dp[r] - dr[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pw[r] = __builtin_amdgcn_exp2f(fmaf(s[r], p.c, -lr[r]));
          ds[r] = pw[r] * (dp[r] - dr[r]);
        }
      }
      bf16x8_t pp[2], pd[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t w1, w2;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          w1[e2] = pack_bf16(pw[8 * ks + 2 * e2], pw[8 * ks + 2 * e2 + 1]);
          w2[e2] = pack_bf16(ds[8 * ks + 2 * e2], ds[8 * ks + 2 * e2 + 1]);
        }
        pp[ks] = __builtin_bit_cast(bf16x8_t, w1);
        pd[ks] = __builtin_bit_cast(bf16x8_t, w2);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8 * DB, 0);
      __builtin_amdgcn_sched_barrier(0);
      // dV^T += dO^T P and dK^T += Q^T dS (A: transpose reads; B: this lane's key)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4_t ad = {td[ks][db][0][0], td[ks][db][0][1], td[ks][db][1][0], td[ks][db][1][1]};
          const u32x4_t aq = {tq[ks][db][0][0], tq[ks][db][0][1], tq[ks][db][1][0], tq[ks][db][1][1]};
          dvt[db] = mfma(__builtin_bit_cast(bf16x8_t, ad), pp[ks], dvt[db]);
          dkt[db] = mfma(__builtin_bit_cast(bf16x8_t, aq), pd[ks], dkt[db]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }

  if (key < s_k) {
    uint16_t* gk = p.dk + ((int64_t)bh * s_k + key) * D;
    uint16_t* gv = p.dv + ((int64_t)bh * s_k + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        u32x2_t wk, wv2;
        wk[0] = pack_bf16(dkt[db][4 * gi + 0] * p.scale, dkt[db][4 * gi + 1] * p.scale);
        wk[1] = pack_bf16(dkt[db][4 * gi + 2] * p.scale, dkt[db][4 * gi + 3] * p.scale);
        wv2[0] = pack_bf16(dvt[db][4 * gi + 0], dvt[db][4 * gi + 1]);
        wv2[1] = pack_bf16(dvt[db][4 * gi + 2], dvt[db][4 * gi + 3]);
        *(u32x2_t*)(gk + 32 * db + 8 * gi + 4 * hl) = wk;
        *(u32x2_t*)(gv + 32 * db + 8 * gi + 4 * hl) = wv2;
      }
  }
}

// ---------------------------------------------------------------------------
// dkv kernel, wave-pair form
// ---------------------------------------------------------------------------
// The same work as attn_bwd_dkv_kernel (one workgroup per (b, h, 128-key
// tile), walking its 128-query tiles), split between two waves per 32 keys.
// The single-wave form keeps K and V fragments and both accumulators of its
// keys, about 430 registers, so one wave runs per SIMD and its vector work
// adds to its matrix time. Here waves w and w + 4 (which share a SIMD) own
// keys 32 w .. +31 of the tile:
//   score side (w):        K fragments; S = Q K^T, P = exp2(S c - lse log2 e)
//                          with the masks, dV^T += dO^T P;
//   gradient side (w + 4): V fragments; dP = dO V^T, dS = P (dP - D) with P
//                          taken from the partner through LDS, dK^T += Q^T dS.
// Each wave holds one fragment set and one accumulator, so two fit a SIMD
// and one's vector work overlaps the other's matrix products. P crosses in
// bf16, the value the dV product uses too. Phase j (closed by a workgroup
// barrier): the score side handles 32-query block j and writes its P to
// exchange slot j % 2; the gradient side forms dS and dK of block j - 1 from
// slot (j - 1) % 2, then dP of block j (kept in registers for the next
// phase). A slot is written in phase j and read in phase j + 1, and the read
// of phase j + 1 precedes the next write of the slot (phase j + 2) by a
// barrier.
template <int D, bool CAUSAL, bool PADMASK>
__global__ __launch_bounds__(512, 2) void attn_bwd_dkv_pair_kernel(BwdParams p) {
  constexpr int NT = 512, BK = 128, BQ = 128;
  constexpr int QB = BQ / 32, DK = D / 16, DB = D / 32;
  constexpr int RB = 2 * D;                   // bytes per Q / dO row in LDS
  constexpr int SL = D / 8;                   // 16-byte slots per row
  constexpr int TILE = BQ * RB;               // one Q or dO tile
  constexpr int BUF = 2 * TILE + 2 * BQ * 4;  // Q, dO, lse*log2e, D
  constexpr int NQ = BQ * SL / NT;            // loads per wave per Q or dO tile
  constexpr int XS = 4 * 64 * 32;             // exchange slot: 4 wave pairs x 64 lanes x 32 bytes
  static_assert((BQ * SL) % NT == 0, "a tile is a whole number of loads per wave");
  static_assert(QB >= 2, "the next tile's loads start in a tile's second block");

  __shared__ __attribute__((aligned(16))) char lds[2 * BUF + 2 * XS];
  char* const xs = lds + 2 * BUF;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pr = wv & 3;       // wave pair: keys 32 pr .. +31 of the tile
  const bool grad = wv >= 4;   // gradient side (dP, dS, dK) or score side (S, P, dV)
  const int hl = lane >> 5, ln = lane & 31;
  const int L = blockIdx.x;
  const int kt = L / p.BH;
  const int bh = L % p.BH, b = bh / p.H;
  const int k0 = kt * BK;
  const int s_q = p.s_q, s_k = p.s_k;

  // key side, one key per lane: K (score side) or V (gradient side) fragments
  const int key = k0 + 32 * pr + ln;
  bf16x8_t kvf[DK];
  {
    const __amdgpu_buffer_rsrc_t r = make_rsrc((grad ? p.v : p.k) + (int64_t)bh * s_k * D, (uint32_t)s_k * D * 2);
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
      kvf[kk] = __builtin_bit_cast(bf16x8_t, load16(r, (uint32_t)(key * D + 16 * kk + 8 * hl) * 2));
  }
  bool kvis = key < s_k;
  if (PADMASK && kvis) kvis = p.kpm[(int64_t)b * s_k + key] == 0;
  // causal: this key is hidden from query qi when kcut > qi (every query
  // when the key itself is hidden)
  const int kcut = kvis ? key : INT_MAX;
  const bool keys_masked = PADMASK || __ballot(!kvis) != 0ull;
  const int kmax = k0 + 32 * pr + 31;  // the pair's last key

  // query tiles that can see a key of this tile; none when every key of the
  // block is padded (its gradients are zero)
  const int qt0 = CAUSAL ? min(k0, s_q) / BQ : 0;
  int qt1 = (s_q + BQ - 1) / BQ;
  if (PADMASK && !__syncthreads_or(kvis)) qt1 = qt0;
  const uint16_t* qg = p.q + (int64_t)bh * s_q * D;
  const uint16_t* dg = p.dout + (int64_t)bh * s_q * D;
  const float* l2g = p.lse2w + (int64_t)bh * p.s_qp;
  const float* Dg = p.delta + (int64_t)bh * p.s_qp;

  // Staging: loads that write LDS directly, untracked by the compiler (it
  // would otherwise wait for them before the next LDS read of any buffer);
  // the barrier before a tile's first use waits for them. Load i of this
  // wave fills LDS slots 64 (8 i + wv) .. +63 of the Q and of the dO tile.
  // Rows past s_q read zeros.
  uint32_t q_voff[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int sl = 64 * (8 * i + wv) + lane;
    const int r = sl / SL, ph = sl % SL;
    q_voff[i] = (uint32_t)(r * RB + 16 * (ph ^ q_swz<D>(r)));
  }
  auto dma_tile = [&](int u, int bi) __attribute__((always_inline)) {
    const int i0 = u * BQ;
    char* base = lds + bi * BUF;
    const uint32_t rest = (uint32_t)max(s_q - i0, 0) * RB;
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      load16_to_lds_untracked(qg + (int64_t)i0 * D, rest, base + 64 * (8 * i + wv) * 16, q_voff[i]);
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      load16_to_lds_untracked(dg + (int64_t)i0 * D, rest, base + TILE + 64 * (8 * i + wv) * 16, q_voff[i]);
    // lse*log2e then D of the tile's BQ rows, BQ / 4 slots each: wave wv < 4
    // loads slots LS (wv & 1) .. +LS-1 of lse*log2e (waves 0, 1) or of D
    // (waves 2, 3). The workspace holds s_qp >= i0 + BQ rows per (b, h).
    constexpr int LS = BQ / 8;
    if (wv < 4 && lane < LS)
      load16_to_lds_untracked((wv < 2 ? l2g : Dg) + i0, BQ * 4, base + 2 * TILE + 16 * LS * wv,
                              (uint32_t)(16 * (LS * (wv & 1) + lane)));
  };

  // Score-side fragment reads (Q for S, dO for dP): lane (ln, hl) reads row
  // key_of_row(ln) of each 32-row block at logical slot 2 kk + hl.
  int a_off[DK];
  {
    const int r = key_of_row(ln);
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) a_off[kk] = r * RB + 16 * ((2 * kk + hl) ^ q_swz<D>(r));
  }
  // Transpose reads of the gradient products' A operands (dO^T for dV, Q^T
  // for dK), as in the single-wave form.
  int t_off[2][DB];
  {
    const int a = lane & 15, g = (lane >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int row = 8 * hl + 4 * r + (a >> 2);
        const int slot = 4 * db + 2 * g + ((a & 3) >> 1);
        t_off[r][db] = row * RB + 16 * (slot ^ q_swz<D>(row)) + 8 * (a & 1);
      }
  }
  // this lane's 32 bytes of a P block in an exchange slot (16 per half)
  const int x_off = pr * 2048 + lane * 16;

  f32x16_t acc[DB];  // dV^T (score side) or dK^T (gradient side)
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};
  f32x16_t dpk = {};  // gradient side: dP of the block whose dS comes next

  // the gradient product of one block: acc[db] += A^T (rows of the block) x w,
  // A^T from transpose reads of the block's rows (grad_reads)
  auto grad_reads = [&](const char* src, int qb, u32x2_t (&t)[2][DB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 2; ++r) t[ks][db][r] = lds_read_tr16(src + t_off[r][db] + (32 * qb + 16 * ks) * RB);
  };
  auto grad_mfma = [&](const u32x2_t (&t)[2][DB][2], const bf16x8_t* w) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4_t a = {t[ks][db][0][0], t[ks][db][0][1], t[ks][db][1][0], t[ks][db][1][1]};
        acc[db] = mfma(__builtin_bit_cast(bf16x8_t, a), w[ks], acc[db]);
      }
  };
  // S (score side) or dP (gradient side) of one block: one key per lane, the
  // registers hold queries 32 qb + {8 hl .. 8 hl + 7, 16 + 8 hl .. +7}
  auto score_reads = [&](const char* src, int qb, bf16x8_t (&f)[DK]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) f[kk] = *(const bf16x8_t*)(src + a_off[kk] + qb * 32 * RB);
  };
  auto score_mfma = [&](const bf16x8_t (&f)[DK]) __attribute__((always_inline)) -> f32x16_t {
    f32x16_t s = {};
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) s = mfma(f[kk], kvf[kk], s);
    return s;
  };
  // The barrier closing a phase, without the wait of a fenced barrier for
  // every LDS access of the wave: the reads of the next phase's operands stay
  // in flight across it (they read a tile that no wave writes before two
  // more barriers have passed). The only LDS writes of a phase, the score
  // side's P, are waited for explicitly before it; the memory clobber keeps
  // the compiler from moving LDS accesses across it.
  auto phase_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  const int n_it = qt1 - qt0;
  const int nb = n_it * QB;  // 32-query blocks
  if (n_it > 0) dma_tile(qt0, 0);
  wait_loads();
  __syncthreads();
  // Each side runs its own loop over the phases (one loop with a branch per
  // side made the compiler copy the accumulators at the join every phase);
  // both take the same barriers.
  auto phase_begin = [&](int j) __attribute__((always_inline)) {
    // the next tile goes to the other buffer once its last reader, the
    // gradient side's block before this tile, has passed a barrier
    const int it = j / QB;
    if (j % QB == 1 && it + 1 < n_it) dma_tile(qt0 + it + 1, (it + 1) & 1);
  };
  auto phase_end = [&](int j) __attribute__((always_inline)) {
    // the next tile's loads have landed before the barrier that precedes its
    // first block
    if (j % QB == QB - 1 && j / QB + 1 < n_it) wait_loads();
    phase_sync();
  };
  // Software pipelining across the barriers: each side requests the LDS
  // operands of its next phase at the end of the current one (after the
  // products that consume the registers), so their latency overlaps the
  // barrier and the other waves' work. A block that starts a new tile is
  // read after the barrier that makes the tile valid; so is P, which the
  // partner writes in the phase before.
  if (!grad) {
    f32x4_t lv[4];           // lse*log2e of the block's rows
    bf16x8_t f[DK];          // Q fragments (S)
    u32x2_t t[2][DB][2];     // dO^T (dV)
    auto loads = [&](int j) __attribute__((always_inline)) {
      const int it = j / QB, qb = j % QB;
      const char* ql = lds + (it & 1) * BUF;
      const float* lw = (const float*)(ql + 2 * TILE);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int qo = 32 * qb + 16 * h2 + 8 * hl;
        lv[2 * h2] = *(const f32x4_t*)(lw + qo);
        lv[2 * h2 + 1] = *(const f32x4_t*)(lw + qo + 4);
      }
      score_reads(ql, qb, f);
      grad_reads(ql + TILE, qb, t);
    };
    for (int j = 0; j <= nb; ++j) {
      phase_begin(j);
      if (j < nb) {
        const int it = j / QB, qb = j % QB;
        if (qb == 0) loads(j);
        __builtin_amdgcn_sched_barrier(0);
        const int qrow = (qt0 + it) * BQ + 32 * qb;
        const f32x16_t s = score_mfma(f);
        float pw[16];
        // masks where a key is hidden, on the causal diagonal, and on the
        // ragged last block (its rows past s_q carry lse = -inf)
        if (keys_masked || (CAUSAL && qrow < kmax) || qrow + 32 > s_q) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float lr = lv[r >> 2][r & 3];
            const int qi = qrow + 16 * (r >> 3) + 8 * hl + (r & 7);
            const bool hide = (lr == -INFINITY) | (CAUSAL ? (kcut > qi) : !kvis);
            pw[r] = __builtin_amdgcn_exp2f(hide ? -INFINITY : fmaf(s[r], p.c, -lr));
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) pw[r] = __builtin_amdgcn_exp2f(fmaf(s[r], p.c, -lv[r >> 2][r & 3]));
        }
        bf16x8_t pp[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4_t w;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) w[e2] = pack_bf16(pw[8 * ks + 2 * e2], pw[8 * ks + 2 * e2 + 1]);
          pp[ks] = __builtin_bit_cast(bf16x8_t, w);
          *(u32x4_t*)(xs + (j & 1) * XS + x_off + 1024 * ks) = w;
        }
        grad_mfma(t, pp);  // dV^T += dO^T P
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): P is in LDS before the barrier
        if (qb + 1 < QB && j + 1 < nb) loads(j + 1);
      }
      phase_end(j);
    }
  } else {
    f32x4_t dv4[4];          // D of the rows of the block whose dS comes next
    u32x2_t t[2][DB][2];     // Q^T of that block (dK)
    bf16x8_t fn[DK];         // dO fragments of the block whose dP comes next
    auto dO_loads = [&](int j) __attribute__((always_inline)) {
      score_reads(lds + ((j / QB) & 1) * BUF + TILE, j % QB, fn);
    };
    for (int j = 0; j <= nb; ++j) {
      phase_begin(j);
      if (j < nb && j % QB == 0) dO_loads(j);
      if (j > 0) {
        const int jb = j - 1;
        u32x4_t pw[2];  // P of block jb, from the partner
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) pw[ks] = *(const u32x4_t*)(xs + (jb & 1) * XS + x_off + 1024 * ks);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8_t pd[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4_t w;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int r = 8 * ks + 2 * e2;
            const float p0 = __builtin_bit_cast(float, pw[ks][e2] << 16);
            const float p1 = __builtin_bit_cast(float, pw[ks][e2] & 0xFFFF0000u);
            w[e2] = pack_bf16(p0 * (dpk[r] - dv4[r >> 2][r & 3]), p1 * (dpk[r + 1] - dv4[(r + 1) >> 2][(r + 1) & 3]));
          }
          pd[ks] = __builtin_bit_cast(bf16x8_t, w);
        }
        grad_mfma(t, pd);  // dK^T += Q^T dS
      } else {
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j < nb) {
        dpk = score_mfma(fn);  // dP = dO V^T
        __builtin_amdgcn_sched_barrier(0);
        // operands of the next phase: D and Q^T of this block (its dS and
        // dK come next), dO of the next block when it is in this tile
        const int it = j / QB, qb = j % QB;
        const char* ql = lds + (it & 1) * BUF;
        const float* lw = (const float*)(ql + 2 * TILE);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int qo = BQ + 32 * qb + 16 * h2 + 8 * hl;
          dv4[2 * h2] = *(const f32x4_t*)(lw + qo);
          dv4[2 * h2 + 1] = *(const f32x4_t*)(lw + qo + 4);
        }
        grad_reads(ql, qb, t);
        if (qb + 1 < QB && j + 1 < nb) dO_loads(j + 1);
      }
      phase_end(j);
    }
  }

  if (key < s_k) {
    uint16_t* g = (grad ? p.dk : p.dv) + ((int64_t)bh * s_k + key) * D;
    const float f = grad ? p.scale : 1.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        u32x2_t w;
        w[0] = pack_bf16(acc[db][4 * gi + 0] * f, acc[db][4 * gi + 1] * f);
        w[1] = pack_bf16(acc[db][4 * gi + 2] * f, acc[db][4 * gi + 3] * f);
        *(u32x2_t*)(g + 32 * db + 8 * gi + 4 * hl) = w;
      }
  }
}

// Zero n 16-bit elements (a degenerate problem's gradients). A kernel rather
// than a memset, so the call can be captured into a graph.
__global__ __launch_bounds__(256) void zero_u16_kernel(uint16_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

hipError_t zero_u16(void* p, int64_t n, hipStream_t s) {
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_u16_kernel, dim3((int)std::max<int64_t>(blocks, 1)), dim3(256), 0, s,
                     (uint16_t*)p, n);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool PADMASK>
hipError_t launch_bwd(const BwdParams& p, int grid_q, int grid_k, hipStream_t s) {
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL, PADMASK>), dim3(grid_q), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (grid_k > 0) {
    if constexpr (D == 128)
      hipLaunchKernelGGL((attn_bwd_dkv_pair_kernel<D, CAUSAL, PADMASK>), dim3(grid_k), dim3(512), 0, s, p);
    else
      hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, CAUSAL, PADMASK>), dim3(grid_k), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

}  // namespace

// Rows of the workspace per (b, h): s_q rounded up to the dkv kernel's 128-row
// query tiles.
static int64_t ws_rows(int64_t s_q) { return (s_q + 127) / 128 * 128; }

extern "C" int64_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t s_q) {
  if (B < 0 || H < 0 || s_q < 0) return -1;
  return (2 * B * H * ws_rows(s_q) * 4 + 255) / 256 * 256;
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d, float scale,
                        int causal, const uint8_t* key_padding_mask, void* workspace,
                        int64_t workspace_bytes, void* stream) {
  if (B < 0 || H < 0 || s_q < 0 || s_k < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  const int64_t kMaxSeq = (int64_t)1 << 22;
  if (s_q > kMaxSeq || s_k > kMaxSeq) return ATTN_ERR_SHAPE;
  if (H > 0 && B > INT32_MAX / H) return ATTN_ERR_SHAPE;
  const int64_t BH = B * H;
  const int64_t n_qt = (s_q + 127) / 128, n_kt = (s_k + 127) / 128;
  if (BH * n_qt > (int64_t)INT32_MAX || BH * n_kt > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  if (BH == 0 || (s_q == 0 && s_k == 0)) return ATTN_OK;
  const bool need_q = s_q > 0, need_k = s_k > 0;
  if (need_q && (!q || !out || !dout || !lse || !dq)) return ATTN_ERR_NULL;
  if (need_k && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL;
  if (need_q && need_k && !workspace) return ATTN_ERR_NULL;
  const uintptr_t al = (uintptr_t)q | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq |
                       (uintptr_t)k | (uintptr_t)v | (uintptr_t)dk | (uintptr_t)dv;
  if (al & 15u) return ATTN_ERR_ALIGN;
  if (((uintptr_t)lse & 3u) || ((uintptr_t)workspace & 255u)) return ATTN_ERR_ALIGN;
  const int64_t need = attn_bwd_workspace_bytes(B, H, s_q);
  if (need_q && need_k && workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  const int64_t nq = BH * s_q * d * 2, nk = BH * s_k * d * 2, nl = BH * s_q * 4;
  const void* ins[7] = {q, k, v, out, dout, lse, key_padding_mask};
  const int64_t nin[7] = {nq, nk, nk, nq, nq, nl, key_padding_mask ? B * s_k : 0};
  void* outs[4] = {dq, dk, dv, workspace};
  const int64_t nout[4] = {nq, nk, nk, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (ranges_overlap(outs[i], nout[i], ins[j], nin[j])) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (ranges_overlap(outs[i], nout[i], outs[j], nout[j])) return ATTN_ERR_ALIAS;
  }
  hipStream_t hs = (hipStream_t)stream;
  if (!need_k) {
    // no keys: every row is empty and every gradient is zero
    const hipError_t e = zero_u16(dq, nq / 2, hs);
    g_last_hip_error = (int)e;
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
  }
  BwdParams p = {};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)out;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.s_qp = (int)ws_rows(s_q);
  p.delta = (float*)workspace;
  p.lse2w = (float*)workspace + BH * p.s_qp;
  p.kpm = key_padding_mask;
  p.s_q = (int)s_q;
  p.s_k = (int)s_k;
  p.H = (int)H;
  p.BH = (int)BH;
  p.n_qt = (int)n_qt;
  p.n_kt = (int)n_kt;
  p.c = scale * kLog2e;
  p.scale = scale;
  const int grid_q = (int)(BH * n_qt);
  const int grid_k = (int)(BH * n_kt);
  const bool pad = key_padding_mask != nullptr;
  hipError_t e;
  if (!need_q) {
    // no queries: dk and dv are zero
    e = zero_u16(dk, nk / 2, hs);
    if (e == hipSuccess) e = zero_u16(dv, nk / 2, hs);
  } else if (d == 128) {
    if (causal)
      e = pad ? launch_bwd<128, true, true>(p, grid_q, grid_k, hs) : launch_bwd<128, true, false>(p, grid_q, grid_k, hs);
    else
      e = pad ? launch_bwd<128, false, true>(p, grid_q, grid_k, hs) : launch_bwd<128, false, false>(p, grid_q, grid_k, hs);
  } else {
    if (causal)
      e = pad ? launch_bwd<64, true, true>(p, grid_q, grid_k, hs) : launch_bwd<64, true, false>(p, grid_q, grid_k, hs);
    else
      e = pad ? launch_bwd<64, false, true>(p, grid_q, grid_k, hs) : launch_bwd<64, false, false>(p, grid_q, grid_k, hs);
  }
  g_last_hip_error = (int)e;
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
