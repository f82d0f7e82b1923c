// attn_unfused.hip - the materialising (unfused) attention forward for gfx950
// and its C ABI: the path the fused kernel avoids, built to measure it.
//
// The onecalc.app page "Attention memory" ("The quadratic term", "What this
// memory is", "The formula") describes it: every query is compared with every
// key, the s_q x s_k score matrix of each (batch item, head) is stored in
// device memory, B*H*s_q*s_k*e bytes with e = 2 for 16-bit scores ("Worked
// example"), turned into weights by a row softmax and multiplied by the value
// rows. The hyper.ai story on PyTorch's attention backends reports the plain
// (Math) backend that does this as several times slower than the fused ones,
// its cost being the traffic of that matrix; and that an out-of-place
// masked_fill makes a hidden copy of it. Here the masks are applied in
// place, inside the softmax, so the path moves the matrix four times and
// never copies it:
//   1. scores:  S = scale * Q K^T, rounded to bf16, written   (2 bytes/score)
//   2. softmax: read S, hide masked keys, write the weights P = softmax(S)
//               (bf16) over S, and the row's log-sum-exp       (2 + 2 bytes)
//   3. values:  read P, O = P V (float32 accumulate, bf16 out) (2 bytes)
// Each kernel streams the matrix once: the path is bound by HBM bandwidth.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"
#include "attn_common.h"

namespace {

using namespace attn_detail;

constexpr int kRows = 128;   // query rows per workgroup (4 waves of 32)
constexpr int kKeysWG = 1024;  // keys per workgroup of the score kernel

// ---------------------------------------------------------------- 1. scores
// Workgroup: 128 query rows x up to 1024 keys of one (b, h), in tiles of 64
// keys. Each wave keeps its 32 queries' Q fragments in registers and computes
// S^T = K Q^T per 32-key block with v_mfma_f32_32x32x16_bf16, K rows fed in
// the key_of_row order so that accumulator registers 0..7 / 8..15 of lane half
// h hold keys 8h..8h+7 / 16+8h..16+8h+7 of its query. The wave's 32 x 64
// block of bf16 scores goes through its own LDS staging area (rows padded by
// 16 bytes) so that the stores to device memory are whole 128-byte row
// segments, 8 rows per instruction, instead of 16-byte pieces of 32 rows. The
// K tile passes through registers into LDS rows padded by 16 bytes
// (conflict-free fragment reads), double-buffered, the next tile's loads in
// flight during the products. VEC (s_k a multiple of 8): 16-byte accesses;
// otherwise 2-byte stores.
template <int D, bool VEC>
__global__ __launch_bounds__(256, 2) void unf_scores_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           uint16_t* __restrict__ S, int s_q,
                                                           int s_k, int n_qt, int n_kc,
                                                           float scale) {
  constexpr int DK = D / 16;
  constexpr int KT = 64;              // keys per tile
  constexpr int KS = D * 2 + 16;      // K row stride in LDS (bytes)
  constexpr int UNITS = KT * D / 8;   // 16-byte units per K tile
  constexpr int UPT = UNITS / 256;    // per thread
  constexpr int SS = KT * 2 + 16;     // staging row stride (bytes)
  __shared__ __attribute__((aligned(16))) char lds[2 * KT * KS + 4 * 32 * SS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, ln = lane & 31;
  const int id = blockIdx.x;
  const int kc = id % n_kc;
  const int qt = (id / n_kc) % n_qt;
  const int bh = id / (n_kc * n_qt);
  const int q0 = qt * kRows;
  const int jc0 = kc * kKeysWG;
  const int jc1 = min(s_k, jc0 + kKeysWG);
  const int n_t = (jc1 - jc0 + KT - 1) / KT;

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + (int64_t)bh * s_q * D, (uint32_t)s_q * D * 2);
  bf16x8_t qf[DK];
  const uint32_t qrow = (uint32_t)(q0 + 32 * w + ln);
#pragma unroll
  for (int kk = 0; kk < DK; ++kk)
    qf[kk] = __builtin_bit_cast(bf16x8_t, load16(rq, (qrow * D + 16 * kk + 8 * hl) * 2));

  const uint16_t* kh = k + (int64_t)bh * s_k * D;
  u32x4_t kr[UPT];
  auto load_tile = [&](int t) {
    const int j0 = jc0 + t * KT;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh + (int64_t)j0 * D, (uint32_t)max(s_k - j0, 0) * D * 2);
#pragma unroll
    for (int u = 0; u < UPT; ++u) kr[u] = load16(rk, (uint32_t)(u * 256 + tid) * 16);
  };
  auto store_tile = [&](int t) {
    char* dst = lds + (t & 1) * KT * KS;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = u * 256 + tid;
      *(u32x4_t*)(dst + (unit / (D / 8)) * KS + (unit % (D / 8)) * 16) = kr[u];
    }
  };

  char* stage = lds + 2 * KT * KS + w * 32 * SS;
  const int k_lane_off = key_of_row(ln) * KS + hl * 16;
  // store phase: lane l writes 16 bytes of row 8 i + l / 8 at column 16 (l % 8)
  const int st_row = lane >> 3, st_col = (lane & 7) * 8;

  if (n_t > 0) load_tile(0);
  for (int t = 0; t < n_t; ++t) {
    store_tile(t);
    __syncthreads();
    if (t + 1 < n_t) load_tile(t + 1);
    const char* kl = lds + (t & 1) * KT * KS + k_lane_off;
    f32x16_t acc[KT / 32];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb) {
        const bf16x8_t a = *(const bf16x8_t*)(kl + kb * 32 * KS + kk * 32);
        acc[kb] = mfma(a, qf[kk], kk ? acc[kb] : f32x16_t{});
      }
    }
    // scaled scores, bf16, into the wave's staging rows (query ln, 8 keys per
    // 16-byte piece); the wave reads them back row-wise below, after its own
    // writes (LDS accesses of one wave complete in order)
#pragma unroll
    for (int kb = 0; kb < KT / 32; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4_t wv;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wv[e] = pack_bf16(acc[kb][8 * half + 2 * e] * scale, acc[kb][8 * half + 2 * e + 1] * scale);
        *(u32x4_t*)(stage + ln * SS + (32 * kb + 16 * half + 8 * hl) * 2) = wv;
      }
    }
    const int jt = jc0 + t * KT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + st_row;
      const int row = q0 + 32 * w + r;
      const u32x4_t wv = *(const u32x4_t*)(stage + r * SS + st_col * 2);
      const int j = jt + st_col;
      if (row < s_q) {
        uint16_t* dst = S + ((int64_t)bh * s_q + row) * s_k + j;
        if (VEC) {
          if (j < s_k) *(u32x4_t*)dst = wv;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (j + e < s_k) dst[e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

// ---------------------------------------------------------------- 2. softmax
// One wave per row of S, in place. A row's elements are read in chunks of 64
// lanes x EPL (8 with VEC: one 16-byte load per lane); the first NC chunks
// stay in registers, later ones are read again in the second and third
// passes. Pass 1: max over visible keys; pass 2: sum of exp(x - max); pass 3:
// P = exp(x - max) / sum, rounded to bf16, written over the scores (0 for a
// hidden key). lse = max + ln(sum); a row with no visible key gets P = 0 and
// lse = -inf.
template <bool VEC>
__global__ __launch_bounds__(256) void unf_softmax_kernel(uint16_t* __restrict__ S,
                                                          float* __restrict__ lse,
                                                          const uint8_t* __restrict__ kpm,
                                                          int64_t rows, int s_q, int s_k, int H,
                                                          int causal) {
  constexpr int EPL = VEC ? 8 : 1;
  constexpr int CH = 64 * EPL;
  constexpr int NC = VEC ? 16 : 32;
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // the whole wave leaves together
  const int64_t bh = r / s_q;
  const int i = (int)(r - bh * s_q);
  const int b = (int)(bh / H);
  uint16_t* srow = S + r * s_k;
  const uint8_t* mrow = kpm ? kpm + (int64_t)b * s_k : nullptr;
  const int nch = (s_k + CH - 1) / CH;
  const int jlim = causal ? min(s_k, i + 1) : s_k;  // keys from jlim on are hidden

  typedef uint32_t chunk_t __attribute__((ext_vector_type(EPL == 8 ? 4 : 1)));
  auto load_chunk = [&](int c, uint32_t& vis) -> chunk_t {
    const int j = c * CH + lane * EPL;
    chunk_t x = {};
    vis = 0u;
    if (VEC) {
      if (j < s_k) {
        x = *(const chunk_t*)(srow + j);
        uint64_t mb = 0;
        if (mrow) mb = *(const uint64_t*)(mrow + j);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          if (j + e < jlim && ((mb >> (8 * e)) & 0xFFu) == 0) vis |= 1u << e;
      }
    } else {
      if (j < s_k) {
        x[0] = srow[j];
        if (j < jlim && (!mrow || mrow[j] == 0)) vis = 1u;
      }
    }
    return x;
  };
  auto elem = [&](const chunk_t& x, int e) -> float {
    const uint32_t wd = VEC ? x[e >> 1] : x[0];
    const uint32_t bits = VEC ? ((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16)) : (wd << 16);
    return __builtin_bit_cast(float, bits);
  };

  chunk_t cache[NC];
  uint32_t cvis[NC];
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch) cache[c] = load_chunk(c, cvis[c]);
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        if ((cvis[c] >> e) & 1u) m = fmaxf(m, elem(cache[c], e));
    }
  for (int c = NC; c < nch; ++c) {
    uint32_t vis;
    const chunk_t x = load_chunk(c, vis);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if ((vis >> e) & 1u) m = fmaxf(m, elem(x, e));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const bool empty = m == -INFINITY;
  const float mc = empty ? 0.f : m * kLog2e;

  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        if ((cvis[c] >> e) & 1u) sum += __builtin_amdgcn_exp2f(fmaf(elem(cache[c], e), kLog2e, -mc));
    }
  for (int c = NC; c < nch; ++c) {
    uint32_t vis;
    const chunk_t x = load_chunk(c, vis);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if ((vis >> e) & 1u) sum += __builtin_amdgcn_exp2f(fmaf(elem(x, e), kLog2e, -mc));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  const float inv = empty ? 0.f : __builtin_amdgcn_rcpf(sum);

  auto write_chunk = [&](int c, const chunk_t& x, uint32_t vis) {
    const int j = c * CH + lane * EPL;
    if (j >= s_k) return;
    float p[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      p[e] = ((vis >> e) & 1u) ? __builtin_amdgcn_exp2f(fmaf(elem(x, e), kLog2e, -mc)) * inv : 0.f;
    if (VEC) {
      chunk_t o;
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) o[e] = pack_bf16(p[2 * e], p[2 * e + 1 < EPL ? 2 * e + 1 : 0]);
      *(chunk_t*)(srow + j) = o;
    } else {
      srow[j] = (uint16_t)(pack_bf16(p[0], 0.f) & 0xFFFFu);
    }
  };
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (c < nch) write_chunk(c, cache[c], cvis[c]);
  for (int c = NC; c < nch; ++c) {
    uint32_t vis;
    const chunk_t x = load_chunk(c, vis);
    write_chunk(c, x, vis);
  }
  if (lane == 0) lse[r] = empty ? -INFINITY : m + __builtin_amdgcn_logf(sum) * kLn2;
}

// ---------------------------------------------------------------- 3. values
// Workgroup: 128 query rows of one (b, h), walking the keys in tiles of 64.
// O^T += V^T P^T with v_mfma_f32_32x32x16_bf16: the B operand (P^T, one
// query per lane, 8 consecutive keys per lane half) is a 16-byte load straight
// from the weight matrix, requested two tiles ahead; the A operand (V^T) is
// read from the V tile in LDS (rows padded by 64 bytes) with 16-bit transpose
// reads, two per fragment. V tiles pass through registers into LDS, double
// buffered. Keys past s_k read as zero weights and zero values.
template <int D, bool VEC>
__global__ __launch_bounds__(256, 2) void unf_values_kernel(const uint16_t* __restrict__ P,
                                                           const uint16_t* __restrict__ v,
                                                           uint16_t* __restrict__ out, int s_q,
                                                           int s_k, int n_qt) {
  constexpr int DB = D / 32;
  constexpr int KT = 64;
  constexpr int RB = D * 2 + 64;
  constexpr int UNITS = KT * D / 8;
  constexpr int UPT = UNITS / 256;
  __shared__ __attribute__((aligned(16))) char lds[2 * KT * RB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 5, ln = lane & 31;
  const int qt = blockIdx.x % n_qt;
  const int bh = blockIdx.x / n_qt;
  const int row = qt * kRows + 32 * w + ln;
  const bool row_ok = row < s_q;
  const uint16_t* prow = P + ((int64_t)bh * s_q + (row_ok ? row : 0)) * s_k;
  const uint16_t* vh = v + (int64_t)bh * s_k * D;
  const int n_t = (s_k + KT - 1) / KT;

  u32x4_t vr[UPT];
  auto load_v = [&](int t) {
    const int j0 = t * KT;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh + (int64_t)j0 * D, (uint32_t)max(s_k - j0, 0) * D * 2);
#pragma unroll
    for (int u = 0; u < UPT; ++u) vr[u] = load16(rv, (uint32_t)(u * 256 + tid) * 16);
  };
  auto store_v = [&](int t) {
    char* dst = lds + (t & 1) * KT * RB;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = u * 256 + tid;
      *(u32x4_t*)(dst + (unit / (D / 8)) * RB + (unit % (D / 8)) * 16) = vr[u];
    }
  };
  // weights of tile t for this lane: keys 64 t + 16 c + 8 hl .. + 7, c = 0..3
  auto load_p = [&](int t, u32x4_t (&pw)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = t * KT + 16 * c + 8 * hl;
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (VEC) {
        if (row_ok && j < s_k) x = *(const u32x4_t*)(prow + j);
      } else if (row_ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (j + e < s_k) x[e >> 1] |= (uint32_t)prow[j + e] << (16 * (e & 1));
      }
      pw[c] = x;
    }
  };

  const int v_lane_off = (8 * hl + ((lane & 15) >> 2)) * RB + 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) +
                         8 * (lane & 1);
  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};
  u32x4_t p0[4], p1[4], p2[4];
  if (n_t > 0) {
    load_v(0);
    load_p(0, p0);
    if (n_t > 1) load_p(1, p1);
  }
  for (int t = 0; t < n_t; ++t) {
    store_v(t);
    __syncthreads();
    if (t + 1 < n_t) load_v(t + 1);
    if (t + 2 < n_t) load_p(t + 2, p2);
    const char* vl = lds + (t & 1) * KT * RB + v_lane_off;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, p0[c]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* a = vl + 16 * c * RB + db * 64;
        const u32x2_t lo = lds_read_tr16(a);
        const u32x2_t hi = lds_read_tr16(a + 4 * RB);
        const u32x4_t av = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = mfma(__builtin_bit_cast(bf16x8_t, av), b, o[db]);
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      p0[c] = p1[c];
      p1[c] = p2[c];
    }
  }
  if (row_ok) {
    uint16_t* og = out + ((int64_t)bh * s_q + row) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2_t wv;
        wv[0] = pack_bf16(o[db][4 * g + 0], o[db][4 * g + 1]);
        wv[1] = pack_bf16(o[db][4 * g + 2], o[db][4 * g + 3]);
        *(u32x2_t*)(og + 32 * db + 8 * g + 4 * hl) = wv;
      }
    }
  }
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

int finish(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_LAUNCH;
  }
  g_last_hip_error = 0;
  return ATTN_OK;
}

template <int D, bool VEC>
hipError_t launch_unfused(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out,
                          float* lse, uint16_t* S, const uint8_t* kpm, int64_t BH, int H, int s_q,
                          int s_k, float scale, int causal, hipStream_t hs) {
  const int n_qt = (s_q + kRows - 1) / kRows;
  const int n_kc = (s_k + kKeysWG - 1) / kKeysWG;
  if (s_k > 0) {
    hipLaunchKernelGGL((unf_scores_kernel<D, VEC>), dim3((unsigned)(BH * n_qt * n_kc)), dim3(256), 0, hs,
                       q, k, S, s_q, s_k, n_qt, n_kc, scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t rows = BH * s_q;
  hipLaunchKernelGGL((unf_softmax_kernel<VEC>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, hs, S, lse,
                     kpm, rows, s_q, s_k, H, causal);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((unf_values_kernel<D, VEC>), dim3((unsigned)(BH * n_qt)), dim3(256), 0, hs, S, v, out,
                     s_q, s_k, n_qt);
  return hipGetLastError();
}

}  // namespace

extern "C" int64_t attn_fwd_unfused_workspace_bytes(int64_t B, int64_t H, int64_t s_q, int64_t s_k) {
  if (B < 0 || H < 0 || s_q < 0 || s_k < 0) return -1;
  if (B == 0 || H == 0 || s_q == 0 || s_k == 0) return 0;
  if (B > INT64_MAX / H) return -1;
  const int64_t rows = B * H;
  if (rows > INT64_MAX / s_q) return -1;
  const int64_t rq = rows * s_q;
  if (rq > INT64_MAX / 2 / s_k) return -1;
  return rq * s_k * 2;
}

extern "C" int attn_fwd_unfused(const void* q, const void* k, const void* v, void* out, float* lse,
                                int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d,
                                float scale, int causal, const uint8_t* key_padding_mask,
                                void* scores, int64_t scores_bytes, void* stream) {
  int st = attn_fwd_validate(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal, key_padding_mask);
  if (st != ATTN_OK) return st;
  if (B * H == 0 || s_q == 0) return ATTN_OK;
  const int64_t need = attn_fwd_unfused_workspace_bytes(B, H, s_q, s_k);
  if (need < 0) return ATTN_ERR_SHAPE;
  const int64_t BH = B * H;
  const int64_t n_qt = (s_q + kRows - 1) / kRows;
  const int64_t n_kc = (s_k + kKeysWG - 1) / kKeysWG;
  if (BH * n_qt * (n_kc > 0 ? n_kc : 1) > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  if ((BH * s_q + 3) / 4 > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  if (need > 0) {
    if (!scores) return ATTN_ERR_NULL;
    if ((uintptr_t)scores & 15u) return ATTN_ERR_ALIGN;
    if (scores_bytes < need) return ATTN_ERR_WORKSPACE;
    const int64_t nq = BH * s_q * d * 2, nk = BH * s_k * d * 2, nl = BH * s_q * 4;
    const void* bufs[6] = {q, k, v, out, lse, key_padding_mask};
    const int64_t sizes[6] = {nq, nk, nk, nq, nl, key_padding_mask ? B * s_k : 0};
    for (int i = 0; i < 6; ++i)
      if (overlaps(scores, need, bufs[i], sizes[i])) return ATTN_ERR_ALIAS;
  }
  // 16-byte score rows and 8-byte mask reads need s_k % 8 == 0 and an 8-byte aligned mask
  const bool vec = (s_k % 8) == 0 && ((uintptr_t)key_padding_mask & 7u) == 0;
  hipStream_t hs = (hipStream_t)stream;
  const uint16_t *qp = (const uint16_t*)q, *kp = (const uint16_t*)k, *vp = (const uint16_t*)v;
  uint16_t *op = (uint16_t*)out, *sp = (uint16_t*)scores;
  const int Hi = (int)H, sq = (int)s_q, sk = (int)s_k;
  hipError_t e;
  if (d == 128)
    e = vec ? launch_unfused<128, true>(qp, kp, vp, op, lse, sp, key_padding_mask, BH, Hi, sq, sk, scale, causal, hs)
            : launch_unfused<128, false>(qp, kp, vp, op, lse, sp, key_padding_mask, BH, Hi, sq, sk, scale, causal, hs);
  else
    e = vec ? launch_unfused<64, true>(qp, kp, vp, op, lse, sp, key_padding_mask, BH, Hi, sq, sk, scale, causal, hs)
            : launch_unfused<64, false>(qp, kp, vp, op, lse, sp, key_padding_mask, BH, Hi, sq, sk, scale, causal, hs);
  return finish(e);
}
