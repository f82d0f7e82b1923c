// attn_common.h - device helpers shared by the forward and backward kernels
// (gfx950, wave64): bf16 MFMA, bf16 packing, buffer resources with range
// checks, buffer-to-LDS loads, and the row permutation that makes a score
// accumulator directly usable as the next product's operand.
#ifndef EXACT_ATTENTION_44_AMD_ATTN_COMMON_H
#define EXACT_ATTENTION_44_AMD_ATTN_COMMON_H

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <atomic>

namespace attn_detail {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));  // 32 E4M3 codes
typedef int i32x2_t __attribute__((ext_vector_type(2)));

// hipError_t behind the calling thread's last ATTN_ERR_LAUNCH (any entry point)
__attribute__((visibility("hidden"))) inline thread_local int g_last_hip_error = 0;

// Compute units of the current device (cached per device; host code): a
// persistent grid has one workgroup per CU. Threads calling at once may each
// query and store the same value; the cache entries are atomic for that.
inline hipError_t cu_count(int* n) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cached[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDev) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *n = c;
      return hipSuccess;
    }
  }
  int v = 0;
  e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (v < 1) v = 1;
  if (dev >= 0 && dev < kMaxDev) cached[dev].store(v, std::memory_order_relaxed);
  *n = v;
  return hipSuccess;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Row of the A operand fed to accumulator row m of a 32x32x16 MFMA so that
// accumulator registers 0..7 of lane half h hold rows 8h..8h+7 and registers
// 8..15 hold rows 16+8h..16+8h+7: exactly the layout of the B operand (eight
// consecutive k per lane half) of a following product that sums over those
// rows.
__device__ __forceinline__ int key_of_row(int m) {
  const int a = m >> 3, hh = (m >> 2) & 1, b = m & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + b;
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32x32x64 product of OCP E4M3 operands with float32 accumulation. Lane L
// holds row (A) or column (B) L % 32 and the 32 consecutive k values
// 32 * (L / 32) .. +31, one code per byte, lowest k in the lowest byte.
__device__ __forceinline__ f32x16_t mfma_e4m3(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four float32 values rounded to E4M3 codes (nearest even; magnitudes from
// 480 up give NaN, so callers keep them below that), first value in the
// lowest byte.
__device__ __forceinline__ uint32_t pack_e4m3(float x0, float x1, float x2, float x3) {
  // the first conversion keeps the upper half of its third operand, which the
  // second one overwrites: any value will do, and x0's bits need no move
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, __builtin_bit_cast(int, x0), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}

// LDS transpose read of 8-bit elements: within each group of 16 lanes, byte
// k (0..7) of lane i comes from the address given by lane 2k + (i >= 8) of
// the group, plus (i & 7). The eight even lanes' 8-byte rows are transposed
// into lanes 0..7 and the odd lanes' rows into lanes 8..15.
__device__ __forceinline__ i32x2_t lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)p);
}

// XOR applied to the 16-byte slot index of row r of a 64-row bf16 tile in LDS
// (V in the forward, K and V in the backward's dq kernel, Q and dO in its dkv
// kernel; unpadded rows of 2D bytes; it depends on r mod 16 only). The score-side
// reads take one slot of 16 rows (a permutation of an aligned group of 16);
// the transpose reads take 4 adjacent slots of 4 adjacent rows per half wave;
// with this permutation both kinds of read hit distinct banks.
template <int D>
__device__ __forceinline__ int q_swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (((r & 2) << 1) | ((r >> 2) & 3));
}

// 16-bit LDS transpose read: within each group of 16 lanes, element k (0..3)
// of lane i = 4j + c comes from the address given by lane 4k + j of the
// group, plus c elements.
__device__ __forceinline__ u32x2_t lds_read_tr16(const char* p) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)p));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Buffer resource over [base, base + bytes): loads past the end return zero,
// which pads ragged query and key tails without branches.
// The fields are wave-uniform by construction; readfirstlane states that to
// the compiler so the descriptor stays in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)n, 0x00020000);
}

// 16 bytes per lane from the buffer straight into LDS: lane i's bytes land at
// dst + 16 i (dst is wave-uniform). A device function of its own, so the host
// compilation pass never sees the LDS address-space cast.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, byte_off, 0,
                                          0, 0);
}

// load16_to_lds for a buffer over [base, base + bytes), issued so that the
// compiler does not track it. The compiler cannot tell which LDS bytes such a
// load writes, so for a tracked load it waits for completion before any later
// LDS read; a kernel that reads other LDS buffers meanwhile uses this form and
// waits itself (wait_loads) before the data is read. The statement has no
// memory clobber either: its destination is read only after a barrier that
// follows such a wait. M0 holds the LDS
// destination; the first s_nop covers a preceding vector write of the
// resource's scalar registers, the second the M0 write.
// (M0 is reserved to the compiler, which therefore does not preserve it across
// the statement; the kernels that use this form keep nothing else in M0.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load16_to_lds_untracked(const void* base, uint32_t bytes, char* dst,
                                                        uint32_t byte_off) {
  const uint64_t a = (uint64_t)base;
  u32x4_t rs;
  rs[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  rs[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xFFFFu;
  rs[2] = __builtin_amdgcn_readfirstlane(bytes);
  rs[3] = 0x00020000u;
  const uint32_t m0 =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)dst);
  asm volatile(
      "s_nop 4\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(byte_off), "s"(rs), "s"(m0)
      : "m0");
}
#pragma clang diagnostic pop

// Wait until every vector-memory load of this wave, untracked ones included,
// has completed (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ u32x4_t load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// Largest number of key tiles whose visibility list build_tile_list keeps.
constexpr int kTileListMax = 4096;

// Visibility of the keys [0, kend) of a work item, from its padding mask
// (mg[j] == 0: key j visible), in BC-key tiles (BC <= 64), n_t of them.
// Returns the number of tiles that hold a visible key, the same in every
// lane, and sets *ka, *kb to the first visible key and one past the last
// (0, 0 when none). When the visible keys are exactly [ka, kb) (padding only
// before and after them, the usual case) *contig is 1 and nothing else is
// written; otherwise *contig is 0 and tl[0 .. count) lists the tiles that
// hold a visible key, in increasing order, followed by 8 zero entries.
// bits: scratch of at least kTileListMax / 8 bytes, 8-byte aligned; scr:
// 3 * NW + 4 ints. Every thread of the workgroup (NW waves) calls it: it
// holds two workgroup barriers. Each wave votes on 8 tiles per step (its lanes
// read one key each, all eight loads in flight together), writing one byte of
// a bitmap and keeping its count of visible keys and their first and last;
// then wave 0 combines the waves' counts and, only when the visible keys are
// not one interval, lists the tiles from the bitmap (lane l: the 64 tiles of
// word l). Requires 0 <= n_t <= kTileListMax and n_t * BC >= kend.
template <int BC, int NW>
__device__ __forceinline__ int build_tile_list(const uint8_t* mg, int kend, int n_t, uint8_t* bits,
                                               uint16_t* tl, int* scr, int* ka, int* kb, int* contig) {
  static_assert(BC <= 64, "one key per lane");
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n_pad = (n_t + 63) & ~63;  // whole bitmap words; bits past n_t are zero
  int nk = 0, lo = INT_MAX, hi = -1;   // this wave's visible keys (wave-uniform)
  for (int s0 = 0; s0 < n_pad; s0 += 8 * NW) {
    const int u0 = s0 + 8 * wv;
    uint32_t mb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) mb[i] = mg[min((u0 + i) * BC + lane, kend - 1)];  // kend >= 1 here
    uint32_t b = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = (u0 + i) * BC + lane;
      const bool vis = lane < BC && u0 + i < n_t && key < kend && mb[i] == 0u;
      const uint64_t v = __ballot(vis);
      if (v != 0ull) {
        b |= 1u << i;
        nk += __popcll(v);
        lo = min(lo, (u0 + i) * BC + (int)__builtin_ctzll(v));
        hi = max(hi, (u0 + i) * BC + 63 - (int)__builtin_clzll(v));
      }
    }
    if (lane == 0 && u0 < n_pad) bits[u0 >> 3] = (uint8_t)b;
  }
  if (lane == 0) {
    scr[3 * wv] = nk;
    scr[3 * wv + 1] = lo;
    scr[3 * wv + 2] = hi;
  }
  __syncthreads();
  if (wv == 0) {
    const int wnk = lane < NW ? scr[3 * lane] : 0;
    int wlo = lane < NW ? scr[3 * lane + 1] : INT_MAX;
    int whi = lane < NW ? scr[3 * lane + 2] : -1;
    int keys = wnk;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      keys += __shfl_xor(keys, off);
      wlo = min(wlo, __shfl_xor(wlo, off));
      whi = max(whi, __shfl_xor(whi, off));
    }
    const bool one_interval = keys == 0 || whi - wlo + 1 == keys;
    const int nw = n_pad / 64;
    const uint64_t word = lane < nw ? *(const uint64_t*)(bits + 8 * lane) : 0ull;
    const int c = __popcll(word);
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int total = __shfl(incl, 63);
    if (!one_interval) {
      int pos = incl - c;
      for (uint64_t wd = word; wd != 0ull; wd &= wd - 1ull) tl[pos++] = (uint16_t)(64 * lane + __builtin_ctzll(wd));
    }
    if (lane == 63) {
      scr[3 * NW] = total;
      scr[3 * NW + 1] = keys ? wlo : 0;
      scr[3 * NW + 2] = keys ? whi + 1 : 0;
      scr[3 * NW + 3] = one_interval ? 1 : 0;
      if (!one_interval) {
#pragma unroll
        for (int e = 0; e < 8; ++e) tl[total + e] = 0;
      }
    }
  }
  __syncthreads();
  *ka = __builtin_amdgcn_readfirstlane(scr[3 * NW + 1]);
  *kb = __builtin_amdgcn_readfirstlane(scr[3 * NW + 2]);
  *contig = __builtin_amdgcn_readfirstlane(scr[3 * NW + 3]);
  return __builtin_amdgcn_readfirstlane(scr[3 * NW]);
}

// Hidden-key bits of the BC-key tile starting at key j0 when the visible keys
// are exactly [ka, kb): bit l set when key j0 + l is outside that range
// (bits past BC are set too). Wave-uniform, scalar arithmetic only.
__device__ __forceinline__ uint64_t hidden_outside(int j0, int ka, int kb) {
  const int lo = min(max(ka - j0, 0), 64), hi = min(max(kb - j0, 0), 64);
  const uint64_t below_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
  const uint64_t below_lo = lo >= 64 ? ~0ull : ((1ull << lo) - 1ull);
  return ~(below_hi & ~below_lo);
}

}  // namespace attn_detail

#endif  // EXACT_ATTENTION_44_AMD_ATTN_COMMON_H
