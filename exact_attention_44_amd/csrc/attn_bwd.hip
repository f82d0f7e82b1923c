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
//               dV^T += dO^T P and dK^T += Q^T dS.
// In both, the rows of the LDS operand are read in the permuted order of
// key_of_row, so the 32x32 accumulators are the bf16 operands of the next
// product after a conversion, with no shuffles. LDS tiles are stored both
// row-major (operands of the score-like products) and transposed (operands of
// the gradient products), the transpose done in registers while storing.
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
  float* delta;        // D = rowsum(dO * O), float32 [B*H][s_q] (workspace)
  const uint8_t* kpm;
  int s_q, s_k, H, BH, n_qt, n_kt;
  float c;             // scale * log2(e): weights are exp2(q.k c - lse log2(e))
  float scale;
};

// LDS tile of BT rows x D columns, stored row-major (row stride 2D+16 bytes)
// and transposed (row stride 2BT+16 bytes). With these strides every 16-lane
// fragment read hits distinct banks and each lane's fragment addresses are a
// base plus immediate offsets.
template <int D, int BT>
struct Tile {
  static constexpr int RS = 2 * D + 16;        // row-major stride
  static constexpr int TS = 2 * BT + 16;       // transposed stride
  static constexpr int ROW_BYTES = BT * RS;
  static constexpr int T_BYTES = D * TS;
  static constexpr int BYTES = ROW_BYTES + T_BYTES;
  // items of 2 rows x 8 columns: loaded as two 16-byte pieces, stored as two
  // row-major pieces and 8 transposed dwords
  static constexpr int ITEMS = (BT / 2) * (D / 8);
};

// Stage items [first, first + n*stride) of one BT x D tile: rows beyond
// `rows` (and all of a tile past the end) read zeros through the range check.
template <int D, int BT, int N>
struct Stager {
  u32x4_t r[N][2];
  __device__ __forceinline__ void load(const uint16_t* base, int rows, int first, int stride) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)max(rows, 0) * D * 2);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int id = first + i * stride;
      if (id < Tile<D, BT>::ITEMS) {
        const int rp = id % (BT / 2), dc = id / (BT / 2);
#pragma unroll
        for (int e = 0; e < 2; ++e) r[i][e] = load16(rs, (uint32_t)((2 * rp + e) * D + 8 * dc) * 2);
      }
    }
  }
  __device__ __forceinline__ void store(char* tile, int first, int stride) const {
    using T = Tile<D, BT>;
    char* tt = tile + T::ROW_BYTES;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int id = first + i * stride;
      if (id < T::ITEMS) {
        const int rp = id % (BT / 2), dc = id / (BT / 2);
#pragma unroll
        for (int e = 0; e < 2; ++e) *(u32x4_t*)(tile + (2 * rp + e) * T::RS + dc * 16) = r[i][e];
        char* dst = tt + (8 * dc) * T::TS + (2 * rp) * 2;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          *(uint32_t*)(dst + c * T::TS) = __builtin_amdgcn_perm(r[i][1][c >> 1], r[i][0][c >> 1], sel);
        }
      }
    }
  }
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
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(BwdParams p) {
  constexpr int NT = 256, BR = 128, BC = 64;
  constexpr int KB = BC / 32, DK = D / 16, DB = D / 32;
  using KT = Tile<D, BC>;                 // K: row-major and transposed
  constexpr int VRS = 2 * D + 16;         // V: row-major only
  constexpr int BUF = KT::BYTES + BC * VRS;
  constexpr int NI = (KT::ITEMS + NT - 1) / NT;  // items per thread

  __shared__ __attribute__((aligned(16))) char lds[2 * BUF];
  __shared__ int lds_last;

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
  if (PADMASK) kend = min(kend, keys_until_last_unpadded(mg, s_k, &lds_last));
  const int n_kv = kend > 0 ? (kend + BC - 1) / BC : 0;

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
  const float lse2 = live ? lse_row * kLog2e : 0.f;
  if (hl == 0 && row < s_q) p.delta[(int64_t)bh * s_q + row] = Dv;

  Stager<D, BC, NI> sk, sv;
  auto load_tile = [&](int u) {
    const int j0 = u * BC;
    sk.load(kg + (int64_t)j0 * D, s_k - j0, tid, NT);
    sv.load(vg + (int64_t)j0 * D, s_k - j0, tid, NT);
  };
  auto store_tile = [&](int u) {
    char* base = lds + (u & 1) * BUF;
    sk.store(base, tid, NT);
    // V row-major only
    char* vl = base + KT::BYTES;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int id = tid + i * NT;
      if (id < KT::ITEMS) {
        const int rp = id % (BC / 2), dc = id / (BC / 2);
#pragma unroll
        for (int e = 0; e < 2; ++e) *(u32x4_t*)(vl + (2 * rp + e) * VRS + dc * 16) = sv.r[i][e];
      }
    }
  };

  f32x16_t dqt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqt[db] = f32x16_t{};
  const int a_off = key_of_row(ln) * KT::RS + hl * 16;  // row-major fragment base
  const int t_off = ln * KT::TS + hl * 16;              // transposed fragment base

  if (n_kv > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < n_kv; ++t) {
    if (t + 1 < n_kv) load_tile(t + 1);
    const char* kl = lds + (t & 1) * BUF;
    const char* ktl = kl + KT::ROW_BYTES;
    const char* vl = kl + KT::BYTES;
    const int j0 = t * BC;
    // S^T = K Q^T and dP^T = V dO^T, one 32-key block at a time
    f32x16_t sc[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16_t a1 = {}, a2 = {};
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) {
        const bf16x8_t fk = *(const bf16x8_t*)(kl + a_off + kb * 32 * KT::RS + kk * 32);
        const bf16x8_t fv = *(const bf16x8_t*)(vl + key_of_row(ln) * VRS + hl * 16 + kb * 32 * VRS + kk * 32);
        a1 = mfma(fk, qf[kk], a1);
        a2 = mfma(fv, df[kk], a2);
      }
      sc[kb] = a1;
      dp[kb] = a2;
    }
    // masks: keys past s_k or padded, and causal (key j hidden from row i when j > i)
    uint64_t hid;
    if (PADMASK) {
      const int key = j0 + lane;
      hid = __ballot(!(key < s_k && mg[key] == 0));
    } else {
      const int rem = s_k - j0;
      hid = rem >= BC ? 0ull : ~((1ull << rem) - 1ull);
    }
    const int lim = row - j0;  // causal: key offset visible iff <= lim
    bf16x8_t pf[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t sh = (uint32_t)(hid >> (32 * kb)) >> (8 * hl);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ko = 32 * kb + 16 * (r >> 3) + 8 * hl + (r & 7);
        const bool hide = !live || ((sh >> (16 * (r >> 3) + (r & 7))) & 1u) || (CAUSAL && ko > lim);
        const float pw = hide ? 0.f : __builtin_amdgcn_exp2f(fmaf(sc[kb][r], p.c, -lse2));
        ds[r] = pw * (dp[kb][r] - Dv);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) w[e2] = pack_bf16(ds[8 * ks + 2 * e2], ds[8 * ks + 2 * e2 + 1]);
        pf[kb][ks] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8_t a = *(const bf16x8_t*)(ktl + t_off + db * 32 * KT::TS + (4 * kb + 2 * ks) * 16);
          dqt[db] = mfma(a, pf[kb][ks], dqt[db]);
        }
    if (t + 1 < n_kv) store_tile(t + 1);
    __syncthreads();
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
__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_kernel(BwdParams p) {
  constexpr int NT = 256, BK = 128, BQ = 64;
  constexpr int QB = BQ / 32, DK = D / 16, DB = D / 32;
  using QTl = Tile<D, BQ>;                // Q and dO: row-major and transposed
  constexpr int BUF = 2 * QTl::BYTES + 2 * BQ * 4;  // Q, dO, lse*log2e, D
  constexpr int NI = (QTl::ITEMS + NT - 1) / NT;

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

  // query tiles that can see a key of this tile
  const int qt0 = CAUSAL ? min(k0, s_q) / BQ : 0;
  const int qt1 = (s_q + BQ - 1) / BQ;
  const uint16_t* qg = p.q + (int64_t)bh * s_q * D;
  const uint16_t* dg = p.dout + (int64_t)bh * s_q * D;
  const float* lg = p.lse + (int64_t)bh * s_q;
  const float* Dg = p.delta + (int64_t)bh * s_q;

  Stager<D, BQ, NI> sq, sd;
  float st_l = 0.f, st_d = 0.f;
  auto load_tile = [&](int u) {
    const int i0 = u * BQ;
    sq.load(qg + (int64_t)i0 * D, s_q - i0, tid, NT);
    sd.load(dg + (int64_t)i0 * D, s_q - i0, tid, NT);
    if (tid < BQ) {
      const int i = i0 + tid;
      const float l = i < s_q ? lg[i] : -INFINITY;
      st_l = l;  // -inf marks a row with no visible key (or past s_q)
      st_d = i < s_q ? Dg[i] : 0.f;
    }
  };
  auto store_tile = [&](int u) {
    char* base = lds + (u & 1) * BUF;
    sq.store(base, tid, NT);
    sd.store(base + QTl::BYTES, tid, NT);
    if (tid < BQ) {
      float* lw = (float*)(base + 2 * QTl::BYTES);
      lw[tid] = st_l == -INFINITY ? -INFINITY : st_l * kLog2e;
      lw[BQ + tid] = st_d;
    }
  };

  f32x16_t dkt[DB], dvt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkt[db] = f32x16_t{};
    dvt[db] = f32x16_t{};
  }
  const int a_off = key_of_row(ln) * QTl::RS + hl * 16;
  const int t_off = ln * QTl::TS + hl * 16;
  const int n_it = qt1 - qt0;

  if (n_it > 0) {
    load_tile(qt0);
    store_tile(qt0);
  }
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    const int u = qt0 + it;
    if (it + 1 < n_it) load_tile(u + 1);
    const char* ql = lds + (u & 1) * BUF;
    const char* qtl = ql + QTl::ROW_BYTES;
    const char* dl = ql + QTl::BYTES;
    const char* dtl = dl + QTl::ROW_BYTES;
    const float* lw = (const float*)(ql + 2 * QTl::BYTES);
    const int i0 = u * BQ;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // S = Q K^T and dP = dO V^T for 32 queries: one key per lane, the
      // registers hold queries 32qb + {8h..8h+7, 16+8h..16+8h+7}
      f32x16_t s = {}, dp = {};
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) {
        const bf16x8_t fq = *(const bf16x8_t*)(ql + a_off + qb * 32 * QTl::RS + kk * 32);
        const bf16x8_t fd = *(const bf16x8_t*)(dl + a_off + qb * 32 * QTl::RS + kk * 32);
        s = mfma(fq, kf[kk], s);
        dp = mfma(fd, vf[kk], dp);
      }
      float lr[16], dr[16];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int qo = 32 * qb + 16 * h2 + 8 * hl;
        const f32x4_t l0 = *(const f32x4_t*)(lw + qo), l1 = *(const f32x4_t*)(lw + qo + 4);
        const f32x4_t d0 = *(const f32x4_t*)(lw + BQ + qo), d1 = *(const f32x4_t*)(lw + BQ + qo + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lr[8 * h2 + e] = l0[e];
          lr[8 * h2 + 4 + e] = l1[e];
          dr[8 * h2 + e] = d0[e];
          dr[8 * h2 + 4 + e] = d1[e];
        }
      }
      float pw[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = i0 + 32 * qb + 16 * (r >> 3) + 8 * hl + (r & 7);
        const bool hide = !kvis || lr[r] == -INFINITY || (CAUSAL && key > qi);
        pw[r] = hide ? 0.f : __builtin_amdgcn_exp2f(fmaf(s[r], p.c, -lr[r]));
        ds[r] = pw[r] * (dp[r] - dr[r]);
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
      // dV^T += dO^T P and dK^T += Q^T dS (A: transposed tiles; B: this lane's key)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = t_off + db * 32 * QTl::TS + (4 * qb + 2 * ks) * 16;
          dvt[db] = mfma(*(const bf16x8_t*)(dtl + off), pp[ks], dvt[db]);
          dkt[db] = mfma(*(const bf16x8_t*)(qtl + off), pd[ks], dkt[db]);
        }
    }
    if (it + 1 < n_it) store_tile(u + 1);
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
  if (grid_k > 0)
    hipLaunchKernelGGL((attn_bwd_dkv_kernel<D, CAUSAL, PADMASK>), dim3(grid_k), dim3(256), 0, s, p);
  return hipGetLastError();
}

bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

}  // namespace

extern "C" int64_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t s_q) {
  if (B < 0 || H < 0 || s_q < 0) return -1;
  return (B * H * s_q * 4 + 255) / 256 * 256;
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
  p.delta = (float*)workspace;
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
