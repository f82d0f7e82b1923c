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
// LDS: K tile row-major [BC][D] with rows padded by 16 bytes, so every
// 16-lane fragment read hits distinct banks; loaded from memory straight into
// LDS (buffer loads with LDS as the destination). The V tile is loaded
// straight into LDS too, row-major [BC][D] with rows padded by 64 bytes, and
// read as the transposed operand V^T by 16-bit LDS transpose reads (the
// padding puts the four rows each half wave reads on disjoint banks, and
// keeps every lane's read addresses one base plus compile-time offsets).
// At D = 64 with a key-padding mask both tiles pass through registers
// instead: K a 16-byte unit per thread, V stored transposed, [D][BC] with
// padded rows, and read by plain fragment reads (measured faster there,
// while without a mask the loads into LDS are faster). Four buffers. The two
// wave groups take
// turns (ping-pong): while one group's waves run the matrix products, the
// other group's waves run the softmax, and each SIMD holds one wave of each
// group, because a wave's own vector instructions do not overlap its own
// MFMAs while those of another wave on the SIMD do. One workgroup barrier
// per key tile keeps the groups in step.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "attn.h"
#include "attn_common.h"

namespace {

using namespace attn_detail;

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;
  const uint8_t* kpm;
  int s_q, s_k, H, BH, n_qt;
  int n_items;      // work items: key chunks x query tiles x (b, h)
  int k_chunk;      // keys per chunk of a key-split launch (a multiple of 64)
  float* o_part;    // key-split partial outputs, fp32 [chunk][B*H][s_q][d]
  float* lse_part;  // key-split partial log-sum-exps, fp32 [chunk][B*H][s_q]
  float c;          // |scale| * log2(e): scores enter exp2 as s * c
  float scale_abs;  // |scale|, for the log-sum-exp output
  uint32_t q_xor;   // 0x80008000 when scale < 0: Q negated, so c stays > 0
  uint32_t q_and;   // 0 when scale == 0: Q zeroed, scores are exactly 0
};

template <int D, bool CAUSAL, bool PADMASK, bool SPLIT>
__global__ __launch_bounds__(512, 2) void attn_fwd_kernel(FwdParams p) {
  constexpr int NT = 512;             // 8 waves: two ping-pong groups of 4
  constexpr int BR = 256;             // query rows per workgroup, 32 per wave
  constexpr int BC = 64;              // keys per tile
  constexpr int KB = BC / 32;         // 32-key blocks per tile
  constexpr int DK = D / 16;          // k-steps of the score product
  constexpr int DB = D / 32;          // 32-column blocks of the output
  constexpr int KU = D / 8;           // 16-byte units per K row
  // LDS rows are padded by 16 bytes: with these strides the 16 lanes of every
  // fragment read hit 16 distinct 4-bank groups, and each lane's fragment
  // addresses are one base plus compile-time offsets.
  // K and V by load-to-LDS, V read by transpose reads; otherwise (D = 64 with
  // a padding mask) both through registers
  constexpr bool VDMA = D == 128 || !PADMASK;
  constexpr int KS = D * 2 + 16;      // K row stride (bytes)
  constexpr int RB = D * 2 + 64;      // V row stride with VDMA (bytes)
  constexpr int VS = BC * 2 + 16;     // V^T row stride otherwise (bytes)
  constexpr int K_BYTES = BC * KS;
  constexpr int BUF_BYTES = K_BYTES + (VDMA ? BC * RB : D * VS);
  constexpr int NBUF = 4;             // see the schedule below
  // Each group stages its half (32 keys) of a tile. With VDMA, K goes from
  // memory straight into its padded LDS rows (buffer loads with LDS as the
  // destination): the half is 32 rows of ROW_SLOTS 16-byte slots, written by
  // K_DMA instructions of 64 consecutive slots each; the last instruction
  // overlaps its predecessor, so the overlap is written twice with the same
  // data, and a padding slot receives its row's first 16 bytes. With VDMA,
  // V's half is 32 rows of RB / 16 slots, written by V_DMA instructions of
  // 64 consecutive slots (a padding slot receives its row's first 16 bytes);
  // otherwise K and V go through registers: K in one 16-byte unit per thread
  // of the group, V in items of 2 keys x 4 columns (one per thread, so every
  // wave stages an equal share), transposed on the way into LDS.
  constexpr int GT = NT / 2;
  constexpr int ROW_SLOTS = KS / 16;
  constexpr int K_SLOTS = 32 * ROW_SLOTS;
  constexpr int K_DMA = (K_SLOTS + 63) / 64;
  constexpr int K_DMA_W = (K_DMA + 3) / 4;  // per wave, at most
  static_assert(K_SLOTS >= 64, "a half tile must fill one DMA instruction");
  constexpr int V_ROW_SLOTS = RB / 16;
  constexpr int V_SLOTS = 32 * V_ROW_SLOTS;
  constexpr int V_DMA = V_SLOTS / 64;
  constexpr int V_DMA_W = (V_DMA + 3) / 4;  // per wave, at most
  static_assert(V_DMA * 64 == V_SLOTS, "a V half tile is a whole number of DMA instructions");
  constexpr int V_ITEMS = 16 * (D / 4);
  constexpr int V_LD = (V_ITEMS + GT - 1) / GT;
  constexpr float kSumLimit = 1048576.f;  // 2^20: see the V step

  __shared__ __attribute__((aligned(16))) char lds[NBUF * BUF_BYTES];
  __shared__ int lds_last;
  // With a padding mask: the key tiles of the current item that hold at least
  // one visible key, in order (followed by 8 zero entries), their count, and
  // a bitmap of tile visibility the list is built from. Items with more than
  // LIST_MAX tiles walk every tile up to the last unpadded key instead.
  constexpr int LIST_MAX = kTileListMax;
  __shared__ uint16_t lds_tl[PADMASK ? LIST_MAX + 8 : 1];
  __shared__ __attribute__((aligned(8))) uint8_t lds_bits[PADMASK ? LIST_MAX / 8 : 8];
  __shared__ int lds_scr[3 * (NT / 64) + 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv >> 2;            // waves w and w+4 share a SIMD
  const int gt = tid & (GT - 1);
  const int hl = lane >> 5;
  const int ln = lane & 31;

  const int s_q = p.s_q, s_k = p.s_k;
  // ---- work items. Item L is (key chunk, query tile, (b, h)) with the
  // (b, h) index fastest, so when B*H is a multiple of 8 every item of a head
  // has the same L mod 8 (the device deals workgroups to its 8 XCDs
  // round-robin, so all of a head's items run on one XCD; an XCD runs 32
  // workgroups at a time, from several heads whose K and V need not fit its
  // L2, and misses are served from the MALL: an order of one head per XCD at
  // a time re-read less but ran slower); causal launches take the longest
  // query tiles first. At D = 128 each workgroup takes one item
  // (L = its index). At D = 64 the grid is persistent (at most one workgroup
  // per CU), which saves the start and end of a workgroup per item (measured
  // +8 % on the padded workload; at D = 128 the loop over items made the
  // compiler's code for the tile loop slower than that saving): workgroup g
  // takes one item per round, g in even rounds and the mirror image of g
  // within its round in odd rounds, keeping g mod 8. Mirrored rounds pair
  // long and short causal tiles, so the workgroups get equal work.
  constexpr bool PERSIST = D == 64;
  const int G = gridDim.x, g = blockIdx.x;
  auto item_of = [&](int round) -> int {
    const int off = (round & 1) ? ((G & 7) == 0 ? G - 8 * (1 + g / 8) + (g & 7) : G - 1 - g) : g;
    return round * G + off;
  };
  struct Item {
    int q0, bh, b, zc, k0, s_kc;
  };
  auto describe = [&](int L) -> Item {
    Item it;
    const int per_chunk = p.n_qt * p.BH;
    it.zc = SPLIT ? L / per_chunk : 0;
    const int Li = SPLIT ? L % per_chunk : L;
    const int qt = CAUSAL ? (p.n_qt - 1 - Li / p.BH) : (Li / p.BH);
    it.q0 = qt * BR;
    it.bh = Li % p.BH;
    it.b = it.bh / p.H;
    // key range: all keys, or chunk zc of a key-split launch; key indices
    // below are relative to k0, s_kc keys are in range
    it.k0 = SPLIT ? it.zc * p.k_chunk : 0;
    it.s_kc = SPLIT ? max(0, min(s_k, it.k0 + p.k_chunk) - it.k0) : s_k;
    return it;
  };
  int round = 0;
  int L_cur = item_of(0);  // < n_items: the grid is at most the item count
  int boff = 0;            // LDS buffer of cur's tile t: (boff + t) % NBUF
  int n_kv = 0;            // key tiles cur walks
  int qlo = 0;             // first query row of this wave in cur
  const uint16_t* kg = nullptr;  // cur's keys and values from k0 on
  const uint16_t* vg = nullptr;
  const uint8_t* mg = nullptr;
  int k0 = 0, s_kc = 0;

  // ---- Q fragments (B operand of the score product), kept in registers.
  bf16x8_t qf[DK];
  auto load_q = [&](const Item& it) {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (int64_t)it.bh * s_q * D, (uint32_t)s_q * D * 2);
    const uint32_t row = (uint32_t)(it.q0 + 32 * wv + ln);
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
      qf[kk] = __builtin_bit_cast(bf16x8_t, load16(rq, (row * D + 16 * kk + 8 * hl) * 2));
  };
  // sign and zero handling of the scale, applied where Q is first used
  auto fix_q = [&]() {
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
      u32x4_t x = __builtin_bit_cast(u32x4_t, qf[kk]);
      x = (x & p.q_and) ^ p.q_xor;
      qf[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  };

  // ---- staging of this group's half (keys 32*grp .. 32*grp+31) of a tile
  const int wg = wv & 3;  // wave within its group
  uint32_t k_voff[K_DMA_W];
#pragma unroll
  for (int i = 0; i < K_DMA_W; ++i) {
    const int j = wg + 4 * i;
    const int slot = min(64 * j, K_SLOTS - 64) + lane;
    const int row = 32 * grp + slot / ROW_SLOTS, un = slot % ROW_SLOTS;
    k_voff[i] = (uint32_t)(row * D + (un < KU ? 8 * un : 0)) * 2;
  }
  // VDMA: K rows of tile u into LDS; completes asynchronously (the next
  // fenced barrier of this wave waits for it).
  // The tile at walk position u of cur is key tile ti (keys ti * BC ..; ti
  // == u except where a padding mask skips tiles); nothing past the walk.
  auto src_tile = [&](const uint16_t* base_cur, int u, int ti, const uint16_t*& src, uint32_t& bytes) -> bool {
    if (u >= n_kv) return false;
    src = base_cur + (int64_t)ti * BC * D;
    bytes = (uint32_t)max(s_kc - ti * BC, 0) * D * 2;
    return true;
  };
  auto dma_k = [&](int u, int ti) {
    const uint16_t* src;
    uint32_t rest;
    if (!src_tile(kg, u, ti, src, rest)) return;
    const __amdgpu_buffer_rsrc_t rkt = make_rsrc(src, rest);
    char* kl = lds + ((boff + u) & (NBUF - 1)) * BUF_BYTES + grp * K_SLOTS * 16;
#pragma unroll
    for (int i = 0; i < K_DMA_W; ++i) {
      const int j = wg + 4 * i;
      if (j < K_DMA) {
        load16_to_lds(rkt, kl + min(64 * j, K_SLOTS - 64) * 16, k_voff[i]);
      }
    }
  };
  // V instructions are dealt starting one wave after K's, so the group's
  // waves issue equal numbers of loads (within one).
  uint32_t v_voff[V_DMA_W];
#pragma unroll
  for (int i = 0; i < V_DMA_W; ++i) {
    const int j = ((wg + 3) & 3) + 4 * i;
    const int slot = 64 * min(j, V_DMA - 1) + lane;
    const int r = 32 * grp + slot / V_ROW_SLOTS, un = slot % V_ROW_SLOTS;
    v_voff[i] = (uint32_t)(r * D + (un < KU ? 8 * un : 0)) * 2;
  }
  // V rows of tile u into LDS, the same way as K (VDMA).
  auto dma_v = [&](int u, int ti) {
    const uint16_t* src;
    uint32_t rest;
    if (!src_tile(vg, u, ti, src, rest)) return;
    const __amdgpu_buffer_rsrc_t rvt = make_rsrc(src, rest);
    char* vl = lds + ((boff + u) & (NBUF - 1)) * BUF_BYTES + K_BYTES + grp * V_SLOTS * 16;
#pragma unroll
    for (int i = 0; i < V_DMA_W; ++i) {
      const int j = ((wg + 3) & 3) + 4 * i;
      if (j < V_DMA) load16_to_lds(rvt, vl + 64 * j * 16, v_voff[i]);
    }
  };
  // V through registers (not VDMA): load_v(u) fetches this thread's item of
  // tile u of cur (zeros past its end), store_v(u) writes it transposed.
  u32x2_t vr[V_LD][2];
  auto load_v = [&](int ti) {
    const int j0 = ti * BC;
    const uint32_t rest = (uint32_t)max(s_kc - j0, 0) * D * 2;
    const __amdgpu_buffer_rsrc_t rvt = make_rsrc(vg + (int64_t)j0 * D, rest);
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int id = i * GT + gt;
      if ((V_ITEMS % GT) == 0 || id < V_ITEMS) {
        const int kq = id & 15, dc = id >> 4;
        const int key = 32 * grp + 2 * kq;
#pragma unroll
        for (int r = 0; r < 2; ++r)
          vr[i][r] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rvt, (int)(((key + r) * D + 4 * dc) * 2), 0, 0));
      }
    }
  };
  // K through registers (not VDMA): each thread of a group holds 16 bytes of
  // one of the group's 32 key rows; load_k(ti) fetches them from key tile ti
  // (zeros past its end), store_k(u) writes them to the K rows of tile u.
  static_assert(VDMA || 32 * KU == GT, "not VDMA: one 16-byte unit of a K half tile per thread");
  u32x4_t kr;  // the K half tile in flight
  auto load_k = [&](int ti) __attribute__((always_inline)) -> u32x4_t {
    const int j0 = ti * BC;
    const uint32_t rest = (uint32_t)max(s_kc - j0, 0) * D * 2;
    const __amdgpu_buffer_rsrc_t rkt = make_rsrc(kg + (int64_t)j0 * D, rest);
    return load16(rkt, (uint32_t)((32 * grp + gt / KU) * D + 8 * (gt % KU)) * 2);
  };
  auto store_k = [&](int u, u32x4_t x) __attribute__((always_inline)) {
    if (u >= n_kv) return;
    char* kl = lds + ((boff + u) & (NBUF - 1)) * BUF_BYTES;
    *(u32x4_t*)(kl + (32 * grp + gt / KU) * KS + 16 * (gt % KU)) = x;
  };
  auto store_v = [&](int u) {
    char* vl = lds + ((boff + u) & (NBUF - 1)) * BUF_BYTES + K_BYTES;
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int id = i * GT + gt;
      if ((V_ITEMS % GT) == 0 || id < V_ITEMS) {
        const int kq = id & 15, dc = id >> 4;
        char* dst = vl + (4 * dc) * VS + (32 * grp + 2 * kq) * 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          *(uint32_t*)(dst + c * VS) = __builtin_amdgcn_perm(vr[i][1][c >> 1], vr[i][0][c >> 1], sel);
        }
      }
    }
  };

  // ---- per-wave running state: O^T (one query per lane), row max, row sum
  f32x16_t o[DB];
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t sc[KB];         // scores of the tile between its two steps
  bf16x8_t pf[KB][2];      // weights of the tile between its two steps
  uint32_t mbyte = 1u;     // this lane's padding byte of the tile in flight
  // Two ways to walk an item, each an instantiation of the tile walk below:
  //  - range (list = std::false_type): the visible keys are exactly
  //    [key_lo, key_hi) (no mask, or padding only before and after them); position u
  //    is key tile toff + u and the hidden keys of a tile follow from key_lo, key_hi
  //    by scalar arithmetic, with no mask reads in the loop;
  //  - list (std::true_type): any other mask. Position u is entry u of the
  //    item's tile list (lds_tl; or key tile u for an item longer than the
  //    list holds), each wave keeps the tiles at positions t .. t + 3 in
  //    lanes 0 .. 3 of one register (t: the tile the next V step handles; a
  //    vector register, as the scalar ones are nearly all in use), and every
  //    tile's mask bytes are read.
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

  const int k_lane_off = key_of_row(ln) * KS + hl * 16;
  // VDMA: transpose-read offset of V^T: read r (0, 1) of feature block db
  // gives keys 8 hl + 4 r .. +3 of a 16-key step for feature 32 db + ln, at
  // v_lane_off + r * 4 * RB + db * 64
  const int v_lane_off = VDMA ? (8 * hl + ((lane & 15) >> 2)) * RB + 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8 * (lane & 1)
                              : ln * VS + hl * 16;
  const float c = p.c;

  // The first LA fragments of each value product are read at the end of the
  // V step before it (see vstep_end), so the M step starts on data that is
  // already in registers instead of waiting for the LDS latency.
  constexpr int LA = 6;               // fragment reads in flight in an M step
  bf16x8_t vpre[LA];
  auto v_frag = [&](int t, int i) -> bf16x8_t {
    // fragment i of tile t's value product: kb = i / 8, ks = (i / 4) & 1, db = i & 3
    const int db = i % DB;
    if constexpr (VDMA) {
      const char* vl = lds + ((boff + t) & (NBUF - 1)) * BUF_BYTES + K_BYTES + v_lane_off + (16 * (i / DB)) * RB + db * 64;
      const u32x2_t lo = lds_read_tr16(vl);
      const u32x2_t hi = lds_read_tr16(vl + 4 * RB);
      const u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
      return __builtin_bit_cast(bf16x8_t, w);
    } else {
      const char* vl = lds + ((boff + t) & (NBUF - 1)) * BUF_BYTES + K_BYTES + v_lane_off;
      return *(const bf16x8_t*)(vl + db * 32 * VS + (i / DB) * 32);
    }
  };
  // M step, first half: O^T += V_t^T P(t)^T.
  auto pv = [&](int t) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t a[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int i = (kb * 2 + ks) * DB + db;
          a[db] = i < LA ? vpre[i < LA ? i : 0] : v_frag(t, i);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = mfma(a[db], pf[kb][ks], o[db]);
      }
  };
  // M step, second half: S(t)^T = K_t Q^T. The key blocks' accumulation
  // chains are interleaved (k-step outer), so consecutive MFMAs never depend
  // on each other's result.
  auto qk = [&](int t, auto list) __attribute__((always_inline)) {
    const char* kl = lds + ((boff + t) & (NBUF - 1)) * BUF_BYTES + k_lane_off;
    f32x16_t acc[KB];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
      bf16x8_t a[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) a[kb] = *(const bf16x8_t*)(kl + kb * 32 * KS + kk * 32);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc[kb] = mfma(a[kb], qf[kk], kk ? acc[kb] : f32x16_t{});
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sc[kb] = acc[kb];
    if constexpr (PADMASK && decltype(list)::value) {
      const int key = tile_at(t, 0, list) * BC + lane;
      mbyte = key < s_kc ? (uint32_t)mg[key] : 1u;
    }
  };
  // One M step: value product of tile tp, then score product of tile tq,
  // software-pipelined so LDS fragment reads run LA fragments ahead of the
  // MFMAs that consume them (an LDS read takes several MFMA durations). With
  // VDMA a value-product fragment takes two transpose reads; otherwise every
  // fragment is one read, and the M step also stages V.
  constexpr int N_PV = KB * 2 * DB;            // value-product MFMAs per M step
  constexpr int N_MF = N_PV + KB * DK;         // MFMAs (= fragments) per M step
  static_assert(LA <= N_PV, "prefetched fragments must belong to the value product");
  auto m_step = [&](int tp, int tq, auto list) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(2);
    pv(tp);
    qk(tq, list);
    if constexpr (!VDMA) {
      store_v(tq + 1);
      load_v(tile_at(tq, 2, list));
      // K(u) is read by group 0 from interval u on: both halves are stored
      // in interval u - 1 (group 0's M(u - 1), group 1's M(u - 2)) and
      // fetched an interval before that
      store_k(tq + 1 + grp, kr);
      kr = load_k(tile_at(tq, 2 + grp, list));
    }
#pragma unroll
    for (int i = 0; i < N_PV - LA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, VDMA ? 2 : 1, 0);  // DS read(s)
    }
#pragma unroll
    for (int i = N_PV - LA; i < N_MF - LA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
    __builtin_amdgcn_sched_barrier(0);  // keep the M step in one piece
    __builtin_amdgcn_s_setprio(0);
  };
  // V step: masks and online softmax of S(t) -> P(t).
  auto vstep = [&](int t, auto list) __attribute__((always_inline)) {
    constexpr bool LIST = decltype(list)::value;
    // the next four list entries, requested before this step's loads into
    // LDS so the compiler has no reason to wait for those loads here
    int ring_new = 0;
    if constexpr (LIST) ring_new = ring_load(t + 1);
    if constexpr (VDMA) {
      dma_k(t + 3, tile_at(t, 3, list));
      dma_v(t + 2, tile_at(t, 2, list));
    }
    const int j0 = tile_at(t, 0, list) * BC;
    // hidden-key bits of the tile (padding, keys past s_k); wave-uniform
    uint64_t hid;
    if constexpr (PADMASK && LIST) {
      hid = __ballot(mbyte != 0u);
    } else {
      hid = hidden_outside(j0, key_lo, key_hi);
    }
    if (hid != 0ull || (CAUSAL && k0 + j0 + BC - 1 > qlo)) {
      const int lim = qlo + ln - k0 - j0;  // causal: key offset visible iff <= lim
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t sh = (uint32_t)(hid >> (32 * kb)) >> (8 * hl);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ko = 32 * kb + 16 * (r >> 3) + 8 * hl + (r & 7);
          const bool hide = ((sh >> (16 * (r >> 3) + (r & 7))) & 1u) || (CAUSAL && ko > lim);
          if (hide) sc[kb][r] = -INFINITY;
        }
      }
    }
    // Reference max: taken from the data on a row's first visible tile (O
    // and l are still zero there). Afterwards it moves only when the tile's
    // exp2 sum shows a score more than ~20 (log2 units) above it, i.e. the
    // sum exceeds 2^20 or overflows; then O and l are rescaled and the tile
    // is recomputed. O / l is the same for any reference.
    // Without a padding mask every row sees key 0, so tile 0 is every row's
    // first visible tile and the test needs no vote.
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
    float nmc = -((m_run == -INFINITY) ? 0.f : m_run) * c;
    // Weights P = exp2(s c - m c): float32 for the row sum, rounded to bf16
    // as the value product's operand. Written as three independent batches
    // (all FMAs, all exp2, then sums and packs) so a lone wave always has an
    // independent instruction to issue instead of waiting on the previous
    // result; the row sum uses four chains.
    auto weights = [&]() -> float {
      float x[KB][16];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[kb][r] = fmaf(sc[kb][r], c, nmc);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[kb][r] = __builtin_amdgcn_exp2f(x[kb][r]);
      // four chains started from the first four weights (0 + w would cost an
      // add: the compiler may not fold it)
      float ps[4] = {x[0][0], x[0][1], x[0][2], x[0][3]};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb > 0 || r >= 4) ps[r & 3] += x[kb][r];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          u32x4_t w;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            w[e2] = pack_bf16(x[kb][8 * ks + 2 * e2], x[kb][8 * ks + 2 * e2 + 1]);
          pf[kb][ks] = __builtin_bit_cast(bf16x8_t, w);
        }
      return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };
    float rs = weights();
    if (__ballot(!(rs <= kSumLimit)) != 0ull) {
      float mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      // a lane whose row has no visible key yet keeps O = l = 0 and the
      // neutral reference (the branch is taken by the whole wave)
      const bool none = m_new == -INFINITY;
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * c);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          o[db][r] *= alpha;
        }
      l_run *= alpha;
      m_run = m_new;
      nmc = none ? 0.f : -m_new * c;
      rs = weights();
    }
    l_run += rs;
    if constexpr (LIST) ringv = ring_new;
  };

  // ---- the workgroup's items, one after the other
  for (;;) {
    const Item cur = describe(L_cur);
    const int L_next = item_of(round + 1);
    const bool has_next = PERSIST && L_next < p.n_items;
    k0 = cur.k0;
    s_kc = cur.s_kc;
    kg = p.k + ((int64_t)cur.bh * s_k + k0) * D;
    vg = p.v + ((int64_t)cur.bh * s_k + k0) * D;
    mg = PADMASK ? p.kpm + (int64_t)cur.b * s_k + k0 : nullptr;
    qlo = cur.q0 + 32 * wv;
    // keys this tile can see: causal stops at the last query row; with a
    // padding mask only the tiles that hold a visible key are walked.
    int kend = s_kc;
    if (CAUSAL) kend = min(kend, cur.q0 + BR - k0);
    const int n_t = kend > 0 ? (kend + BC - 1) / BC : 0;
    toff = 0;
    key_lo = 0;
    key_hi = s_kc;
    use_list = false;
    list_identity = false;
    if (PADMASK && n_t <= LIST_MAX) {
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
      for (int cend = s_kc; cend > 0; cend -= NT * 4) {
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
    load_q(cur);
    // the first tiles' loads (positions 0 .. 2, and without VDMA group 1's K
    // of position 3); selects rather than a branch on the kind of walk
    if (PADMASK) ringv = ring_load(0);
    auto first_tile = [&](int k) -> int {
      return (PADMASK && use_list) ? __builtin_amdgcn_readlane(ringv, k) : toff + k;
    };
    if (n_kv > 0) {
      if constexpr (VDMA) {
        dma_k(0, first_tile(0));
        dma_k(1, first_tile(1));
        dma_k(2, first_tile(2));
        dma_v(0, first_tile(0));
        dma_v(1, first_tile(1));
      } else {
        // K(0), K(1) (and group 1's half of K(2), which its first interval,
        // without an M step, cannot store) now; the next K half in flight
        const u32x4_t k0 = load_k(first_tile(0)), k1 = load_k(first_tile(1)), k2 = load_k(first_tile(2));
        kr = grp == 1 ? load_k(first_tile(3)) : k2;
        store_k(0, k0);
        store_k(1, k1);
        if (grp == 1) store_k(2, k2);
        load_v(first_tile(0));
        store_v(0);
        load_v(first_tile(1));
        store_v(1);
        load_v(first_tile(2));
      }
    }
    __syncthreads();
    fix_q();
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};
    m_run = -INFINITY;
    l_run = 0.f;
    mbyte = 1u;

    // ---- ping-pong schedule: n_kv + 2 intervals, each closed by a workgroup
    // barrier. M(t) = [PV(t-1), QK(t)] issues matrix-core work (and, without
    // VDMA, the register staging of K and V), V(t) = [VDMA: K and V
    // staging; softmax of S(t)] vector-ALU work. Interval 0:
    // group 0 runs QK(0). Interval t + 1 (t < n_kv): group 0 runs V(t) then
    // M(t + 1), group 1 runs M(t) then V(t) (M(n_kv) is PV(n_kv - 1) alone).
    // Interval n_kv + 1: group 1 runs PV(n_kv - 1). Waves w and w + 4 share a
    // SIMD, so while one is in its M step the other is in its V step and the
    // two units overlap; within an interval the two waves switch kinds without
    // a barrier, which saves one barrier per tile over a barrier at every
    // switch.
    // LDS buffer u % 4 holds tile u. Its K part is written in interval u - 2
    // (VDMA: load-to-LDS in V(u - 3)) or u - 1 (stores in group 0's M(u - 1)
    // and group 1's M(u - 2), fetched into registers an interval before) and
    // read by QK(u) in intervals u (group 0) and u + 1 (group 1). Its V part is written in interval u - 1 (VDMA:
    // load-to-LDS in V(u - 2); otherwise stores in M(u - 1), group 0 in
    // interval u - 1 and group 1 in interval u) and read from the prefetch at
    // the end of V(u) (interval u + 1) to PV(u) of group 1 (interval u + 2).
    // So every write comes after the last read of tile u - 4 (K: interval
    // u - 3, V: interval u - 2), and the fenced barrier closing the interval of
    // a write waits for it (loads into LDS included) before any read.
    // The scheduling fences also keep register-only work in its step
    // (otherwise the compiler sinks the softmax into the next M step to fill
    // MFMA gaps, and each wave ends up doing both kinds of work serially).
    auto phase_sync = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    // End of V(t): the first LA fragments of PV(t) are requested here, so their
    // latency overlaps the switch to the M step.
    auto vstep_end = [&](int t) {
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int i = 0; i < LA; ++i) vpre[i] = v_frag(t, i);
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
        pv(n_kv - 1);
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
        pv(n_kv - 1);
        phase_sync();
      }
    };
    if (n_kv > 0) {
      if (PADMASK && use_list)
        walk(std::true_type{});
      else
        walk(std::false_type{});
    }

    // ---- epilogue: O = O^T / l, lse = m * |scale| + ln(l)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
    const int row = qlo + ln;
    if (SPLIT && row < s_q) {
      // partial result of this key chunk: fp32 O / l and its log-sum-exp
      const int64_t pr = ((int64_t)cur.zc * p.BH + cur.bh) * s_q + row;
      float* op = p.o_part + pr * D;
  #pragma unroll
      for (int db = 0; db < DB; ++db) {
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4_t w;
  #pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = o[db][4 * g + e] * inv;
          *(f32x4_t*)(op + 32 * db + 8 * g + 4 * hl) = w;
        }
      }
      if (hl == 0) {
        p.lse_part[pr] = l_tot > 0.f ? m_run * p.scale_abs + __builtin_amdgcn_logf(l_tot) * kLn2
                                     : -INFINITY;
      }
    } else if (row < s_q) {
      uint16_t* og = p.out + ((int64_t)cur.bh * s_q + row) * D;
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
        p.lse[(int64_t)cur.bh * s_q + row] = lse;
      }
    }
    if (!has_next) break;
    boff = (boff + n_kv) & (NBUF - 1);
    L_cur = L_next;
    ++round;
  }
}

// Rows of queries per workgroup (8 waves x 32).
template <int D>
constexpr int rows_per_block() {
  return 256;
}


template <int D, bool CAUSAL, bool PADMASK, bool SPLIT>
hipError_t launch(const FwdParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, PADMASK, SPLIT>), dim3(grid), dim3(512), 0, stream, p);
  return hipGetLastError();
}

// Launch over p.n_items work items (set here from the item count).
template <bool SPLIT>
hipError_t launch_fwd(FwdParams p, int64_t d, bool causal, bool pad, int64_t items, hipStream_t hs) {
  // one workgroup per item at d = 128, a persistent grid at d = 64
  int n_cu = 0;
  if (d == 64) {
    const hipError_t e = cu_count(&n_cu);
    if (e != hipSuccess) return e;
  }
  p.n_items = (int)items;
  const int grid = (int)(d == 64 && items > n_cu ? n_cu : items);
  if (d == 128) {
    if (causal)
      return pad ? launch<128, true, true, SPLIT>(p, grid, hs) : launch<128, true, false, SPLIT>(p, grid, hs);
    return pad ? launch<128, false, true, SPLIT>(p, grid, hs) : launch<128, false, false, SPLIT>(p, grid, hs);
  }
  if (causal)
    return pad ? launch<64, true, true, SPLIT>(p, grid, hs) : launch<64, true, false, SPLIT>(p, grid, hs);
  return pad ? launch<64, false, true, SPLIT>(p, grid, hs) : launch<64, false, false, SPLIT>(p, grid, hs);
}

// Merge of the key-split partial results (one wave per query row): with
// per-chunk log-sum-exps lse_z and outputs O_z (each normalised by its own
// row sum), lse = ln sum_z exp(lse_z) and O = sum_z exp(lse_z - lse) O_z.
// This is the softmax over the union of the chunks' keys (the weights of
// chunk z are its own weights times exp(lse_z - lse)). A row that sees no key
// in any chunk gets O = 0 and lse = -inf. Memory-bound: it reads the
// partials once.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ o_part,
                                                         const float* __restrict__ lse_part,
                                                         uint16_t* __restrict__ out,
                                                         float* __restrict__ lse, int64_t rows,
                                                         int chunks) {
  constexpr int E = D / 64;  // output elements per lane
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;  // the whole wave leaves together
  float m = -INFINITY;
  for (int z = lane; z < chunks; z += 64) m = fmaxf(m, lse_part[(int64_t)z * rows + row]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  uint16_t* orow = out + row * D + lane * E;
  if (m == -INFINITY) {
#pragma unroll
    for (int e = 0; e < E; ++e) orow[e] = 0;
    if (lane == 0) lse[row] = -INFINITY;
    return;
  }
  float s = 0.f;
  for (int z = lane; z < chunks; z += 64)
    s += __builtin_amdgcn_exp2f((lse_part[(int64_t)z * rows + row] - m) * kLog2e);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  const float L = m + __builtin_amdgcn_logf(s) * kLn2;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int z = 0; z < chunks; ++z) {
    const float w = __builtin_amdgcn_exp2f((lse_part[(int64_t)z * rows + row] - L) * kLog2e);
    const float* op = o_part + ((int64_t)z * rows + row) * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(w, op[e], acc[e]);
  }
  if (E == 2) {
    *(uint32_t*)orow = pack_bf16(acc[0], acc[E - 1]);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) orow[e] = (uint16_t)(pack_bf16(acc[e], 0.f) & 0xFFFFu);
  }
  if (lane == 0) lse[row] = L;
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
  // the work items (B * H * query tiles) must fit a 32-bit int
  if (blocks_for(BH, s_q, d) > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
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

namespace {

FwdParams make_params(const void* q, const void* k, const void* v, void* out, float* lse,
                      int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d, float scale,
                      const uint8_t* key_padding_mask) {
  FwdParams p = {};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.out = (uint16_t*)out;
  p.lse = lse;
  p.kpm = key_padding_mask;
  p.s_q = (int)s_q;
  p.s_k = (int)s_k;
  p.H = (int)H;
  p.BH = (int)(B * H);
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
  return p;
}

int finish(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_LAUNCH;
  }
  g_last_hip_error = 0;
  return ATTN_OK;
}

constexpr int64_t kMaxChunks = 65535;

// Keys per chunk for n chunks: a multiple of the 64-key tile.
int64_t chunk_keys(int64_t s_k, int64_t n) {
  const int64_t per = (s_k + n - 1) / n;
  return ((per + 63) / 64) * 64;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                        int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d, float scale,
                        int causal, const uint8_t* key_padding_mask, void* stream) {
  const int st = attn_fwd_validate(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal,
                                   key_padding_mask);
  if (st != ATTN_OK) return st;
  if (B * H == 0 || s_q == 0) return ATTN_OK;
  const FwdParams p = make_params(q, k, v, out, lse, B, H, s_q, s_k, d, scale, key_padding_mask);
  const bool pad = key_padding_mask != nullptr && s_k > 0;
  return finish(launch_fwd<false>(p, d, causal != 0, pad, blocks_for(B * H, s_q, d), (hipStream_t)stream));
}

extern "C" int64_t attn_fwd_split_workspace_bytes(int64_t B, int64_t H, int64_t s_q, int64_t d,
                                                  int64_t n_splits) {
  if (B < 0 || H < 0 || s_q < 0 || (d != 64 && d != 128) || n_splits < 1 ||
      n_splits > kMaxChunks)
    return -1;
  if (n_splits == 1) return 0;
  const int64_t rows = B * H * s_q;
  return align256(n_splits * rows * d * 4) + align256(n_splits * rows * 4);
}

namespace {

// Key-split forward over `chunks` (>= 2) chunks with the partial results in
// `workspace` (at least attn_fwd_split_workspace_bytes(..., chunks) bytes,
// 256-byte aligned, checked by the callers): the chunked forward, then the
// merge, both on `hs`.
int split_launch(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                 int64_t H, int64_t s_q, int64_t s_k, int64_t d, float scale, int causal,
                 const uint8_t* key_padding_mask, int64_t chunks, void* workspace, hipStream_t hs) {
  const int64_t BH = B * H;
  FwdParams p = make_params(q, k, v, out, lse, B, H, s_q, s_k, d, scale, key_padding_mask);
  p.k_chunk = (int)chunk_keys(s_k, chunks);
  p.o_part = (float*)workspace;
  p.lse_part = (float*)((char*)workspace + align256(chunks * BH * s_q * d * 4));
  const bool pad = key_padding_mask != nullptr;
  int st = finish(launch_fwd<true>(p, d, causal != 0, pad, blocks_for(BH, s_q, d) * chunks, hs));
  if (st != ATTN_OK) return st;
  const int64_t rows = BH * s_q;
  const int mgrid = (int)((rows + 3) / 4);
  if (d == 128)
    hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(mgrid), dim3(256), 0, hs, p.o_part, p.lse_part,
                       (uint16_t*)out, lse, rows, (int)chunks);
  else
    hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(mgrid), dim3(256), 0, hs, p.o_part, p.lse_part,
                       (uint16_t*)out, lse, rows, (int)chunks);
  return finish(hipGetLastError());
}

// The chunk count a key-split call uses for n_splits requested chunks: at most
// one per 64-key tile, and at least one.
int64_t split_chunks(int64_t s_k, int64_t n_splits) {
  const int64_t tiles = (s_k + 63) / 64;
  return n_splits < tiles ? n_splits : (tiles > 0 ? tiles : 1);
}

// Host checks of a key-split call with `chunks` >= 2 that do not depend on
// the workspace: grid sizes of the chunked launch and of the merge.
int split_shape_ok(int64_t BH, int64_t s_q, int64_t d, int64_t chunks) {
  if (((BH * s_q + 3) / 4) > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  // work items of the chunked launch: chunks x B * H x query tiles
  if (blocks_for(BH, s_q, d) * chunks > (int64_t)INT32_MAX) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd_split(const void* q, const void* k, const void* v, void* out, float* lse,
                              int64_t B, int64_t H, int64_t s_q, int64_t s_k, int64_t d,
                              float scale, int causal, const uint8_t* key_padding_mask,
                              int64_t n_splits, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  int st = attn_fwd_validate(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal,
                             key_padding_mask);
  if (st != ATTN_OK) return st;
  if (n_splits < 1 || n_splits > kMaxChunks) return ATTN_ERR_SHAPE;
  // fewer chunks than 64-key tiles would leave chunks empty
  const int64_t chunks = split_chunks(s_k, n_splits);
  if (chunks == 1) return attn_fwd(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal,
                                   key_padding_mask, stream);
  const int64_t need = attn_fwd_split_workspace_bytes(B, H, s_q, d, chunks);
  if (B * H == 0 || s_q == 0) return ATTN_OK;
  if (!workspace) return ATTN_ERR_NULL;
  if ((uintptr_t)workspace & 255u) return ATTN_ERR_ALIGN;
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  const int64_t BH = B * H;
  const int64_t nq = BH * s_q * d * 2, nk = BH * s_k * d * 2, nl = BH * s_q * 4;
  const void* bufs[6] = {q, k, v, out, lse, key_padding_mask};
  const int64_t sizes[6] = {nq, nk, nk, nq, nl, key_padding_mask ? B * s_k : 0};
  for (int i = 0; i < 6; ++i)
    if (overlaps(workspace, need, bufs[i], sizes[i])) return ATTN_ERR_ALIAS;
  st = split_shape_ok(BH, s_q, d, chunks);
  if (st != ATTN_OK) return st;
  return split_launch(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal, key_padding_mask,
                      chunks, workspace, (hipStream_t)stream);
}

// ---- the key-split forward without a caller workspace: its partial results
// go to a fixed device array of ATTN_SPLIT_SCRATCH_BYTES bytes (one copy per
// device, held until the process ends), for callers that cannot allocate.
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each device's copy comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is passed
// to kernels.
static __device__ __align__(256) char scratch[ATTN_SPLIT_SCRATCH_BYTES];

namespace {

// Device address of the current device's `scratch` (cached per device).
hipError_t scratch_address(void** out) {
  constexpr int kMaxDev = 64;
  static std::atomic<void*> cached[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDev) {
    void* c = cached[dev].load(std::memory_order_acquire);
    if (c != nullptr) {
      *out = c;
      return hipSuccess;
    }
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (ptr == nullptr) return hipErrorInvalidSymbol;
  if (dev >= 0 && dev < kMaxDev) cached[dev].store(ptr, std::memory_order_release);
  *out = ptr;
  return hipSuccess;
}

}  // namespace

extern "C" int attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* out,
                                      float* lse, int64_t B, int64_t H, int64_t s_q, int64_t s_k,
                                      int64_t d, float scale, int causal,
                                      const uint8_t* key_padding_mask, int64_t n_splits,
                                      void* stream) {
  int st = attn_fwd_validate(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal,
                             key_padding_mask);
  if (st != ATTN_OK) return st;
  if (n_splits < 1 || n_splits > kMaxChunks) return ATTN_ERR_SHAPE;
  const int64_t chunks = split_chunks(s_k, n_splits);
  if (chunks == 1) return attn_fwd(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal,
                                   key_padding_mask, stream);
  if (B * H == 0 || s_q == 0) return ATTN_OK;
  // the partial results must fit the fixed array (checked before any HIP call)
  if (attn_fwd_split_workspace_bytes(B, H, s_q, d, chunks) > (int64_t)ATTN_SPLIT_SCRATCH_BYTES)
    return ATTN_ERR_WORKSPACE;
  st = split_shape_ok(B * H, s_q, d, chunks);
  if (st != ATTN_OK) return st;
  void* ws = nullptr;
  st = finish(scratch_address(&ws));
  if (st != ATTN_OK) return st;
  return split_launch(q, k, v, out, lse, B, H, s_q, s_k, d, scale, causal, key_padding_mask,
                      chunks, ws, (hipStream_t)stream);
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
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: the workspace (or the fixed scratch array) is smaller than required";
    default: return "unknown attn status";
  }
}

extern "C" int attn_last_hip_error(void) { return g_last_hip_error; }
