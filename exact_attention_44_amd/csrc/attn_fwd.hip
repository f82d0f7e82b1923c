// attn_fwd.hip - fused attention forward for gfx950 (CDNA4) and its C ABI.
//
// Method (news.hamidun.com glossary "Flash attention", second paragraph;
// onecalc.app "Attention memory", section "FlashAttention"): keys and values
// are walked in blocks that fit on-chip memory, a running row max m and row
// sum l are kept per query row, each new block rescales what was accumulated
// by exp(m_old - m_new), and the output is normalised once at the end. The
// s_q x s_k score matrix never leaves registers.
//
// Work decomposition (the glossary's note that the second version of the
// method parallelises over the sequence dimension): one workgroup per
// (batch item, head, tile of BR query rows); NW waves per workgroup, each wave
// owns 32 query rows, two waves share a SIMD so one's softmax overlaps the
// other's matrix products.
//
// Register layout. The score tile is computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 features, B = 16 features x 32
// queries). In the 32x32 accumulator, lane L holds column L%32 (one query row)
// and 16 rows (keys); the two wave halves hold different keys of the same
// query. Row max and row sum are therefore in-lane, plus one exchange between
// lanes L and L^32. K rows are read in a permuted order so that accumulator
// registers 0..7 of half h are keys 8h..8h+7 and registers 8..15 are keys
// 16+8h..16+8h+7: exactly the B-operand layout of the next product,
// O^T += V^T P^T, so P goes from the score accumulator to the MFMA operand by
// a bf16 conversion only. The output accumulator O^T has one query row per
// lane too, so the rescale by exp(m_old - m_new) is a per-lane scalar.
//
// LDS: K tile row-major [BC][D], V tile transposed [D][BC] (the transpose is
// done in registers while storing), both with an XOR swizzle of 16-byte units
// so the 16 lanes that share an LDS cycle hit distinct banks. Two buffers: the
// next tile's global loads are issued before the current tile's math, stored
// after it, one barrier per tile.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;  // see the online-softmax step in the kernel

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  const uint8_t* kpm;
  int s_q, s_k, H, BH, n_qt;
  float c;          // |scale| * log2(e): scores enter exp2 as s * c
  float scale_abs;  // |scale|, for the log-sum-exp output
  uint32_t q_xor;   // 0x80008000 when scale < 0: Q negated, so c stays > 0
  uint32_t q_and;   // 0 when scale == 0: Q zeroed, scores are exactly 0
};

// XOR swizzle of 16-byte units for a row of U units. Rows of 256 B (U = 16)
// permute by row & 15; narrower rows by the row's index within 256 B groups,
// so any 16 consecutive rows read at one logical unit touch 16 distinct
// 4-bank groups.
template <int U>
__device__ __forceinline__ int swz(int row) {
  static_assert(U == 4 || U == 8 || U == 16, "unsupported LDS row width");
  return (row / (16 / U)) & (U - 1);
}

// Key row fed to accumulator row m of the score MFMA (see file comment).
__device__ __forceinline__ int key_of_row(int m) {
  const int a = m >> 3, hh = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + b;
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Buffer resource over [base, base + bytes): loads past the end return zero,
// which pads ragged query and key tails without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

template <int D, int NW, int KB, bool CAUSAL, bool PADMASK>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BR = 32 * NW;         // query rows per workgroup, 32 per wave
  constexpr int BC = 32 * KB;         // keys per tile
  constexpr int DK = D / 16;          // k-steps of the score product
  constexpr int DB = D / 32;          // 32-column blocks of the output
  constexpr int KU = D / 8;           // 16-byte units per K row
  constexpr int VU = BC / 8;          // 16-byte units per V^T row
  constexpr int K_BYTES = BC * D * 2;
  constexpr int BUF_BYTES = 2 * K_BYTES;
  constexpr int K_LD = BC * KU / NT;  // 16-byte K loads per thread per tile
  static_assert((BC * KU) % NT == 0, "K tile must split evenly over the threads");
  // V is staged in items of VK keys x 8 columns (VK 16-byte loads, 8 LDS writes)
  constexpr int VK = ((BC / 2) * (D / 8) > NT) ? 4 : 2;
  constexpr int V_ITEMS = (BC / VK) * (D / 8);
  constexpr int V_LD = (V_ITEMS + NT - 1) / NT;
  constexpr int MB = (BC + 63) / 64;  // 64-key mask ballots per tile

  __shared__ __attribute__((aligned(16))) char lds[2 * BUF_BYTES];
  __shared__ int lds_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int ln = lane & 31;

  const int L = blockIdx.x;
  const int qt = CAUSAL ? (p.n_qt - 1 - L / p.BH) : (L / p.BH);
  const int bh = L % p.BH;
  const int b = bh / p.H;
  const int q0 = qt * BR;
  const int s_q = p.s_q, s_k = p.s_k;

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (int64_t)bh * s_q * D, (uint32_t)s_q * D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (int64_t)bh * s_k * D, (uint32_t)s_k * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (int64_t)bh * s_k * D, (uint32_t)s_k * D * 2);
  const uint8_t* mg = PADMASK ? p.kpm + (int64_t)b * s_k : nullptr;

  // ---- keys this tile can see: causal stops at the last query row; padding
  // stops after the last key that is not padded.
  int kend = s_k;
  if (CAUSAL) kend = min(kend, q0 + BR);
  if (PADMASK) {
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
  }
  const int n_kv = (kend + BC - 1) / BC;

  // ---- Q fragments (B operand of the score product), kept in registers.
  bf16x8_t qf[DK];
  {
    const uint32_t row = (uint32_t)(q0 + 32 * wv + ln);
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
      u32x4_t x = load16(rq, (row * D + 16 * kk + 8 * hl) * 2);
      x = (x & p.q_and) ^ p.q_xor;
      qf[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  // ---- tile staging: global -> registers -> LDS
  u32x4_t kr[K_LD];
  u32x4_t vr[V_LD][VK];
  uint32_t mbyte[MB];
  uint64_t cur_mask[MB], next_mask[MB];
#pragma unroll
  for (int t = 0; t < MB; ++t) cur_mask[t] = next_mask[t] = 0;

  auto load_tile = [&](int jt) {
    const int j0 = jt * BC;
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int id = i * NT + tid;
      const int row = id / KU, u = id % KU;
      kr[i] = load16(rk, ((uint32_t)(j0 + row) * D + 8 * u) * 2);
    }
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int id = i * NT + tid;
      if ((V_ITEMS % NT) == 0 || id < V_ITEMS) {
        const int kq = id % (BC / VK), dc = id / (BC / VK);
#pragma unroll
        for (int r = 0; r < VK; ++r)
          vr[i][r] = load16(rv, ((uint32_t)(j0 + VK * kq + r) * D + 8 * dc) * 2);
      }
    }
    if (PADMASK) {
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        const int kl = 64 * t + lane, key = j0 + kl;
        mbyte[t] = (kl < BC && key < s_k) ? (uint32_t)mg[key] : 1u;
      }
    }
  };

  auto store_tile = [&](int buf) {
    char* kl = lds + buf * BUF_BYTES;
    char* vl = kl + K_BYTES;
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int id = i * NT + tid;
      const int row = id / KU, u = id % KU;
      *(u32x4_t*)(kl + row * (KU * 16) + ((u ^ swz<KU>(row)) << 4)) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int id = i * NT + tid;
      if ((V_ITEMS % NT) == 0 || id < V_ITEMS) {
        const int kq = id % (BC / VK), dc = id / (BC / VK);
        // Threads of one column chunk fill one V^T row; the next chunk's rows
        // are 8 further down. Odd chunks walk their 8 rows in swapped pairs so
        // neighbouring chunks write rows of opposite parity (other bank half).
        const int odd = dc & 1;
        const uint32_t sel_even = odd ? 0x07060302u : 0x05040100u;
        const uint32_t sel_odd = odd ? 0x05040100u : 0x07060302u;
        const int key_byte = VK * kq * 2;  // byte offset of this item's keys in a row
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int w = c >> 1;
          const uint32_t sel = (c & 1) ? sel_odd : sel_even;
          const int row = 8 * dc + (c ^ odd);
          char* dst = vl + row * (VU * 16) + (((key_byte >> 4) ^ swz<VU>(row)) << 4) + (key_byte & 15);
          if (VK == 4) {
            u32x2_t val;
            val[0] = __builtin_amdgcn_perm(vr[i][1][w], vr[i][0][w], sel);
            val[1] = __builtin_amdgcn_perm(vr[i][3 % VK][w], vr[i][2 % VK][w], sel);
            *(u32x2_t*)dst = val;
          } else {
            *(uint32_t*)dst = __builtin_amdgcn_perm(vr[i][1][w], vr[i][0][w], sel);
          }
        }
      }
    }
    if (PADMASK) {
#pragma unroll
      for (int t = 0; t < MB; ++t) next_mask[t] = __ballot(mbyte[t] != 0u);
    }
  };

  // ---- running statistics and output accumulator (O^T, one query per lane)
  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  const int k_lane_row = key_of_row(ln);
  const float c = p.c;
  const float lazy_thr = kLazy / c;  // kLazy in log2 units, as a raw-score margin
  const int qlo = q0 + 32 * wv;      // first query row of this wave

  if (n_kv > 0) {
    load_tile(0);
    store_tile(0);
#pragma unroll
    for (int t = 0; t < MB; ++t) cur_mask[t] = next_mask[t];
  }
  __syncthreads();

  for (int jt = 0; jt < n_kv; ++jt) {
    const int buf = jt & 1;
    const bool has_next = jt + 1 < n_kv;
    if (has_next) load_tile(jt + 1);

    const char* kl = lds + buf * BUF_BYTES;
    const char* vl = kl + K_BYTES;
    const int j0 = jt * BC;

    // Hidden-key bits per 32-key block (padding and keys past s_k). These and
    // the causal test below are wave-uniform: interior tiles take no masking
    // branch at all.
    uint32_t mw[KB];
    bool any_mw = false;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (PADMASK) {
        mw[kb] = (uint32_t)(cur_mask[kb >> 1] >> (32 * (kb & 1)));
      } else {
        const int rem = s_k - (j0 + 32 * kb);
        mw[kb] = rem >= 32 ? 0u : (rem <= 0 ? ~0u : ~((1u << rem) - 1u));
      }
      any_mw = any_mw || (mw[kb] != 0u);
    }

    // S^T = K Q^T
    f32x16_t s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int row = 32 * kb + k_lane_row;
      bf16x8_t a[DK];
#pragma unroll
      for (int kk = 0; kk < DK; ++kk)
        a[kk] = *(const bf16x8_t*)(kl + row * (KU * 16) + (((2 * kk + hl) ^ swz<KU>(row)) << 4));
      s[kb] = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) s[kb] = mfma(a[kk], qf[kk], s[kb]);
    }

    // masks
    if (CAUSAL && j0 + BC - 1 > qlo) {
      const int lim = qlo + ln - j0;  // key offset in tile visible iff <= lim
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = 32 * kb + 16 * (r >> 3) + 8 * hl + (r & 7);
          if (ko > lim) s[kb][r] = -INFINITY;
        }
    }
    if (any_mw) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t sh = mw[kb] >> (8 * hl);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((sh >> (16 * (r >> 3) + (r & 7))) & 1u) s[kb][r] = -INFINITY;
      }
    }

    // online softmax
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy reference: move m only when the block max passes it by more than
    // kLazy (log2 units). Weights exp2((s - m) c) then stay <= 2^kLazy and the
    // final O / l is unchanged, while the output rescale becomes a rare,
    // wave-uniform branch (always skipped on the row's first visible block,
    // where O and l are still zero).
    const bool move = mx > m_run + lazy_thr;
    const float m_new = move ? mx : m_run;
    const float alpha = move ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.f;
    const bool rescale = move && (m_run != -INFINITY);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float nmc = -m_ref * c;
    float rs = 0.f;
    bf16x8_t pf[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, nmc));
        rs += e;
        s[kb][r] = e;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t w;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          w[e2] = pack_bf16(s[kb][8 * ks + 2 * e2], s[kb][8 * ks + 2 * e2 + 1]);
        pf[kb][ks] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__ballot(rescale) != 0ull) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t a[DB];
        const int u = 4 * kb + 2 * ks + hl;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int row = 32 * db + ln;
          a[db] = *(const bf16x8_t*)(vl + row * (VU * 16) + ((u ^ swz<VU>(row)) << 4));
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma(a[db], pf[kb][ks], o[db]);
      }
    }

    if (has_next) {
      store_tile(buf ^ 1);
#pragma unroll
      for (int t = 0; t < MB; ++t) cur_mask[t] = next_mask[t];
    }
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, lse = m * |scale| + ln(l)
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
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
      const float lse = l_tot > 0.f
                            ? m_run * p.scale_abs + __builtin_amdgcn_logf(l_tot) * kLn2
                            : -INFINITY;
      p.lse[(int64_t)bh * s_q + row] = lse;
    }
  }
}

// Tile shape per head dimension: NW waves of 32 query rows, KB blocks of 32 keys.
template <int D>
struct Cfg;
template <>
struct Cfg<128> {
  static constexpr int NW = 8, KB = 2;
};
template <>
struct Cfg<64> {
  static constexpr int NW = 8, KB = 2;
};

template <int D>
constexpr int rows_per_block() {
  return 32 * Cfg<D>::NW;
}

template <int D>
constexpr int threads_per_block() {
  return 64 * Cfg<D>::NW;
}

thread_local int g_last_hip_error = 0;

template <int D, bool CAUSAL, bool PADMASK>
hipError_t launch(const FwdParams& p, int grid, hipStream_t stream) {
  using C = Cfg<D>;
  hipLaunchKernelGGL((attn_fwd_kernel<D, C::NW, C::KB, CAUSAL, PADMASK>), dim3(grid),
                     dim3(C::NW * 64), 0, stream, p);
  return hipGetLastError();
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

int64_t blocks_for(int64_t BH, int64_t s_q, int64_t d) {
  const int64_t br = d == 128 ? rows_per_block<128>() : rows_per_block<64>();
  return BH * ((s_q + br - 1) / br);
}

}  // namespace

extern "C" int attn_fwd_validate(const void* q, const void* k, const void* v, const void* out,
                                 const float* lse, int64_t B, int64_t H, int64_t s_q,
                                 int64_t s_k, int64_t d, float scale, int causal,
                                 const uint8_t* key_padding_mask) {
  (void)causal;
  if (B < 0 || H < 0 || s_q < 0 || s_k < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  // one (b, h) slice of q, k or v must stay below 2 GiB (32-bit buffer offsets)
  const int64_t kMaxSeq = (int64_t)1 << 22;
  if (s_q > kMaxSeq || s_k > kMaxSeq) return ATTN_ERR_SHAPE;
  if (H > 0 && B > INT32_MAX / H) return ATTN_ERR_SHAPE;
  const int64_t BH = B * H;
  // the grid's work-items must fit 32 bits
  if (blocks_for(BH, s_q, d) > (int64_t)(UINT32_MAX / 512)) return ATTN_ERR_SHAPE;
  if (BH == 0 || s_q == 0) return ATTN_OK;
  if (!q || !out || !lse) return ATTN_ERR_NULL;
  if (s_k > 0 && (!k || !v)) return ATTN_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)out) & 15u) return ATTN_ERR_ALIGN;
  if (s_k > 0 && (((uintptr_t)k | (uintptr_t)v) & 15u)) return ATTN_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return ATTN_ERR_ALIGN;
  const int64_t nq = BH * s_q * d * 2, nk = BH * s_k * d * 2, nl = BH * s_q * 4;
  const int64_t nm = key_padding_mask ? B * s_k : 0;
  const void* ins[4] = {q, k, v, key_padding_mask};
  const int64_t ns[4] = {nq, nk, nk, nm};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(out, nq, ins[i], ns[i]) || overlaps(lse, nl, ins[i], ns[i])) return ATTN_ERR_ALIAS;
  }
  if (overlaps(out, nq, lse, nl)) return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                        int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d, float scale,
                        int causal, const uint8_t* key_padding_mask, void* stream) {
  const int st = attn_fwd_validate(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal,
                                   key_padding_mask);
  if (st != ATTN_OK) return st;
  const int64_t BH = B * H;
  if (BH == 0 || s_q == 0) return ATTN_OK;

  FwdParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.kpm = key_padding_mask;
  p.s_q = (int)s_q;
  p.s_k = (int)s_k;
  p.H = (int)H;
  p.BH = (int)BH;
  const int64_t br = d == 128 ? rows_per_block<128>() : rows_per_block<64>();
  p.n_qt = (int)((s_q + br - 1) / br);
  const float sa = fabsf(scale);
  if (sa < 1e-30f) {  // exp(scale * q.k) == 1 in float32 for any representable score
    p.q_and = 0u;
    p.q_xor = 0u;
    p.c = kLog2e;
    p.scale_abs = 0.f;
  } else {
    p.q_and = ~0u;
    p.q_xor = scale < 0.f ? 0x80008000u : 0u;
    p.c = sa * kLog2e;
    p.scale_abs = sa;
  }
  const int grid = (int)blocks_for(BH, s_q, d);
  const bool pad = key_padding_mask != nullptr && s_k > 0;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e;
  if (d == 128) {
    if (causal)
      e = pad ? launch<128, true, true>(p, grid, hs) : launch<128, true, false>(p, grid, hs);
    else
      e = pad ? launch<128, false, true>(p, grid, hs) : launch<128, false, false>(p, grid, hs);
  } else {
    if (causal)
      e = pad ? launch<64, true, true>(p, grid, hs) : launch<64, true, false>(p, grid, hs);
    else
      e = pad ? launch<64, false, true>(p, grid, hs) : launch<64, false, false>(p, grid, hs);
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_LAUNCH;
  }
  g_last_hip_error = 0;
  return ATTN_OK;
}

extern "C" const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL: a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE: a size is negative or too large";
    case ATTN_ERR_HEAD_DIM: return "ATTN_ERR_HEAD_DIM: d must be 64 or 128";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN: q/k/v/out need 16-byte, lse 4-byte alignment";
    case ATTN_ERR_ALIAS: return "ATTN_ERR_ALIAS: out or lse overlaps another buffer";
    case ATTN_ERR_SCALE: return "ATTN_ERR_SCALE: scale is NaN or infinite";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH: the HIP runtime refused the launch";
    default: return "unknown attn status";
  }
}

extern "C" int attn_last_hip_error(void) { return g_last_hip_error; }
