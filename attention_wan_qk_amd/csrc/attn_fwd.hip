// Softmax attention forward on bf16 MFMA (gfx950), used for both the full
// self-attention over all video tokens and the cross-attention to text.
//
// Follows the self-attention call of the "Wan2.2 code walkthrough" page,
// flash_attention(q, k, v, k_lens, window_size = (-1, -1)): global window,
// no causal mask, keys at or past k_lens[b] excluded. The L x L score matrix
// is never stored: each workgroup owns 256 query rows of one (batch, head)
// and streams the keys in tiles of 64 with a running (online) softmax.
//
// Layout of the work (per workgroup: 8 wavefronts x 32 query rows, two per
// SIMD):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16. K (A operand, keys x dims) is
//    read from LDS; Q (B operand) stays in registers for the whole loop. In
//    the accumulator each lane owns one query row (lane % 32) and 16 keys, so
//    the row max needs one half-wave swap (v_permlane32_swap) and the row sum
//    none until the end.
//  * O^T += V^T P^T on the same MFMA. P comes straight from the score
//    registers (converted to bf16); V^T is read from the row-major V tile with
//    ds_read_b64_tr_b16, whose key order is chosen to match P's.
//  * Ping-pong: waves 0-3 and 4-7 run the same phase sequence one phase
//    apart (GEMM phase: P V of tile j-1 then S of tile j; softmax phase of
//    tile j), separated by workgroup barriers, so each SIMD always hosts one
//    wave feeding the MFMA pipe while the other runs the softmax on the VALU.
//  * Inside a GEMM phase the LDS operand reads are issued a few fragments
//    ahead of their MFMAs (scheduling groups), hiding LDS latency.
//  * The running max m is in log2 units of the scaled scores and is only
//    moved (O and l rescaled) when a row's tile max exceeds it by more than
//    8, so every P stays <= 2^8 and the rescale is rare. The tile max itself
//    is only formed on a row's first tile and when a lane's sum of P over
//    the tile (32 values) exceeds 2^8, which any exponent above 8 causes;
//    such a tile is recomputed after the rescale. The softmax phase is
//    otherwise one fma, one exp2 and one add per score and the bf16
//    conversion.
//  * K/V tiles are double-buffered in LDS and moved by buffer loads whose
//    destination is the LDS (no register staging), issued at the start of a
//    softmax phase (which reads no LDS): group 1 loads the next K tile and
//    awaits it at the end of its following GEMM phase (the tile is only
//    needed one interval later), group 0 the next V tile, awaited at the end
//    of the softmax phase. The four slots are separate LDS arrays, so the
//    compiler places no wait for a load in flight before the reads of
//    another slot. Rows past k_len fall outside the buffer resource and read
//    as zero. Each 16-byte chunk of a row is
//    XOR-swizzled so the MFMA operand reads are bank-conflict free; a load
//    writes 16 bytes per lane at base + 16 lane, so each lane fetches the
//    global chunk that belongs there.
//  * Workgroup ids are remapped so that each XCD works through consecutive
//    query tiles of the same (batch, head) and shares its K/V in its L2.
//  * The output rows leave through LDS: each wave stages its normalised
//    32 x 128 block and stores whole 256-byte row segments, 4 rows per store
//    instruction (the accumulator layout alone would give 16-byte pieces of
//    32 rows per instruction), which matters for the cross-attention items of
//    only a few key tiles.
//  * With a workspace (self-attention), the work items of the last, partly
//    filled round of the chip are split into key ranges run by otherwise idle
//    CUs; each range leaves its unnormalised output, running max and sum, and
//    a second kernel combines them (the partial softmax results of disjoint
//    key sets merge exactly through their maxima).
#include <mutex>

#include "wan_device.h"
#include "wan_internal.h"

namespace wan {

namespace {

constexpr int kWaves = 8;                    // two groups of four, one wave of each per SIMD
constexpr int kAheadV = 4;                   // V fragments read ahead of their MFMAs
constexpr int kAheadK = 4;                   // K fragments read ahead of their MFMAs
constexpr int kBM = 32 * kWaves;             // query rows per workgroup
constexpr int kBN = 64;                      // keys per tile
static_assert(kBM == kAttnRows && kBN == kAttnKeys, "tiling shared with the host-side planning");
constexpr int kKB = kBN / 32;                // 32-key blocks per tile
constexpr int kKC = kBN / 16;                // 16-key chunks per tile (PV k-steps)
constexpr int kHD = 128;                     // head size
constexpr int kRowBytes = kHD * 2;
constexpr int kTileBytes = kBN * kRowBytes;
constexpr int kThreads = 64 * kWaves;
// 1 KiB tile loads per tile and wave of the loading group
constexpr int kLoadsPerWave = kTileBytes / 1024 / (kWaves / 2);
constexpr float kRescaleThreshold = 8.0f;    // log2 units
constexpr float kSumLimit = 256.0f;          // per-lane tile sum of P that forces the tile max
constexpr uint32_t kRsrcWord3 = 0x00020000u; // raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100;

template <int N>
struct Int {
  static constexpr int value = N;
};

// s_waitcnt vmcnt(0): wait for this wave's outstanding buffer loads only.
constexpr int kWaitLoads = 0x0F70;

// Barrier between phases, without a memory fence. The only LDS writes inside
// the main loop are the buffer loads into LDS; the waves that issue them wait
// for them (kWaitLoads) before the barrier that publishes them. Every LDS
// read of a phase feeds an MFMA issued before that phase's barrier, so it has
// completed. The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x8 lds_read16(const char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ s16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// K tile: 16-byte chunk ch of key row r lives at chunk ch ^ (r % 16), so the
// 16 keys read together at one logical chunk hit 16 different bank groups.
__device__ __forceinline__ int k_phys(int r, int ch) { return ch ^ (r & 15); }
// V tile: a transposed read touches 4 consecutive keys x 4 consecutive
// chunks per half-wave, so the chunk is XORed with 4 * (r % 4).
__device__ __forceinline__ int v_phys(int r, int ch) { return ch ^ ((r & 3) << 2); }

}  // namespace

// kKind: 0 self-attention, 1 cross-attention (same code; separate names in
// profiles), 2 chunk-causal self-attention (per-row key limit, see below).
template <int kKind>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(AttnArgs a) {
  // K and V tiles, slots 0 and 1, each an array of its own: the compiler then
  // knows that a tile load in flight into one slot does not write what the
  // LDS reads of another slot read, and places no wait before those reads.
  __shared__ __attribute__((aligned(1024))) char k_slot0[kTileBytes], k_slot1[kTileBytes],
      v_slot0[kTileBytes], v_slot1[kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int group = wave / (kWaves / 2);    // 0: leads, 1: one phase behind
  const int r32 = lane & 31;
  const int hf = lane >> 5;

  const int nQ = (a.Lq + kBM - 1) / kBM;
  const uint32_t total = (uint32_t)a.B * a.H * nQ;
  // Cross-attention workgroups are persistent (the grid has at most 256 of
  // them, one per CU): with only a few key tiles per query tile, launching a
  // workgroup per tile costs a noticeable share of its short life. The other
  // kinds run one item per workgroup.
  const bool kSplitting = kKind == 0 && a.part != nullptr;
  for (uint32_t item = blockIdx.x;;) {
    // Key-split workgroups (after the n_full whole items) take range
    // split % n_split of item n_full + split / n_split.
    const int split = kSplitting && item >= a.n_full ? (int)(item - a.n_full) : -1;
    const uint32_t logical = split >= 0 ? a.n_full + split / a.n_split
                                        : xcd_remap(item, kSplitting ? a.n_full : total);
    const int qt = logical % nQ;
    const int bh = logical / nQ;
    const int h = bh % a.H;
    const int b = bh / a.H;

    int kv_len = a.Lk;
    if (a.k_lens) kv_len = min(max(a.k_lens[b], 0), a.Lk);
    // Chunk-causal: query row r (global position q_offset + r) sees keys below
    // min(kv_len, (chunk(q_offset + r) + 1) * chunk_len). The workgroup streams
    // the tiles its last row needs and masks per row beyond its first row's limit.
    constexpr bool kCausal = kKind == 2;
    auto key_limit = [&](int row) {
      if (!kCausal) return kv_len;
      const int64_t c = ((int64_t)a.q_offset + row) / a.chunk_len + 1;
      return (int)min((int64_t)kv_len, c * a.chunk_len);
    };
    const int lim_lo = key_limit(min(qt * kBM, a.Lq - 1));
    const int lim_hi = key_limit(min(qt * kBM + kBM - 1, a.Lq - 1));
    // This workgroup streams key tiles t0 .. t0 + nT - 1.
    int t0 = 0, nT = (lim_hi + kBN - 1) / kBN;
    if (split >= 0) {
      const int sp = split % a.n_split, all = nT;
      t0 = (int)((int64_t)all * sp / a.n_split);
      nT = (int)((int64_t)all * (sp + 1) / a.n_split) - t0;
    }

    const uint16_t* qg = static_cast<const uint16_t*>(a.q) + (int64_t)b * a.Lq * a.ld_q + h * kHD;
    const uint16_t* kg = static_cast<const uint16_t*>(a.k) + (int64_t)b * a.Lk * a.ld_k + h * kHD;
    const uint16_t* vg = static_cast<const uint16_t*>(a.v) + (int64_t)b * a.Lk * a.ld_v + h * kHD;
    const uint32_t row_k = (uint32_t)a.ld_k * 2, row_v = (uint32_t)a.ld_v * 2;
    // Bytes of valid keys behind each base: anything past them reads as 0.
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)kg, (short)0, (int)(kv_len * row_k), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)vg, (short)0, (int)(kv_len * row_v), kRsrcWord3);

    // The four waves of a group move a K or V tile from global memory straight
    // into LDS (buffer loads with the LDS as destination). Load i of wave w
    // (w = wave % 4) fills tile rows 4(kLoadsPerWave w + i) .. +3: lane l
    // writes physical chunk l % 16 of row 4(kLoadsPerWave w + i) + l / 16, so
    // it fetches the logical chunk (l % 16) ^ swizzle of that row.
    uint32_t vo_k[kLoadsPerWave], vo_v[kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int r = ((wave & 3) * kLoadsPerWave + i) * 4 + (lane >> 4);
      const int p = lane & 15;
      vo_k[i] = r * row_k + (k_phys(r, p) << 4);  // k_phys is an involution
      vo_v[i] = r * row_v + (v_phys(r, p) << 4);
    }
    auto dma_k = [&](int t, auto slotc) {
      char* const dst = decltype(slotc)::value ? k_slot1 : k_slot0;
      const uint32_t sk = (uint32_t)(t0 + t) * kBN * row_k;
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (lds_void*)(dst + ((wave & 3) * kLoadsPerWave + i) * 1024), 16, vo_k[i], sk, 0, 0);
    };
    auto dma_v = [&](int t, auto slotc) {
      char* const dst = decltype(slotc)::value ? v_slot1 : v_slot0;
      const uint32_t sv = (uint32_t)(t0 + t) * kBN * row_v;
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (lds_void*)(dst + ((wave & 3) * kLoadsPerWave + i) * 1024), 16, vo_v[i], sv, 0, 0);
    };
    // Q fragment: B operand of S^T = K Q^T, lane holds Q[row][16c + 8hf .. +8].
    const int qrow = qt * kBM + wave * 32 + r32;
    const int lim_row = key_limit(min(qrow, a.Lq - 1));
    bf16x8 qf[8];
    {
      const uint16_t* qr = qg + (int64_t)min(qrow, a.Lq - 1) * a.ld_q + 8 * hf;
#pragma unroll
      for (int c = 0; c < 8; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qr + 16 * c);
    }

    if (nT > 0 && group == 0) dma_k(0, Int<0>{});
    __builtin_amdgcn_s_waitcnt(0);   // Q and K tile 0 have landed
    __syncthreads();

    // LDS read addresses (byte offsets inside a tile; the slot, the 32-key
    // block and the key chunk are immediate offsets).
    int ka[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) ka[c] = r32 * kRowBytes + (k_phys(r32, 2 * c + hf) << 4);
    const int g16 = lane >> 4, e4 = (lane & 15) >> 2, q4 = lane & 3;
    int va[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
      va[db] = (4 * (g16 >> 1) + e4) * kRowBytes +
               ((4 * (db ^ e4) + 2 * (g16 & 1) + (q4 >> 1)) << 4) + 8 * (q4 & 1);

    f32x16 oacc[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[d][v] = 0.f;
    float m_used = -INFINITY;
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
    f32x16 s[kKB];
    bf16x8 pf[kKC];

    // GEMM phase of tile jj: O^T += V^T P^T for tile jj - 1 (V slot 1 - KS),
    // then S^T = K Q^T for tile jj (K slot KS).
    auto gemm = [&](auto ksc, int jj) {
      constexpr int KS = decltype(ksc)::value;
      if (jj >= 1 && jj <= nT) {
        const char* Vt = KS ? v_slot0 : v_slot1;
        s16x4 lo[4 * kKC], hi[4 * kKC];
#pragma unroll
        for (int kc = 0; kc < kKC; ++kc) {
          const int krow = 32 * (kc >> 1) + 16 * (kc & 1);
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            lo[kc * 4 + db] = lds_read_tr(Vt + va[db] + krow * kRowBytes);
            hi[kc * 4 + db] = lds_read_tr(Vt + va[db] + (krow + 8) * kRowBytes);
          }
        }
#pragma unroll
        for (int kc = 0; kc < kKC; ++kc) {
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const s16x8 cat =
                __builtin_shufflevector(lo[kc * 4 + db], hi[kc * 4 + db], 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, cat), pf[kc], oacc[db], 0, 0, 0);
          }
        }
        // issue order: kAheadV fragments, then one MFMA per fragment read
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, kAheadV * 2, 0);
#pragma unroll
        for (int i = 0; i < 4 * kKC - kAheadV; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSgMfma, kAheadV, 0);
      }
      if (jj < nT) {
        const char* Kt = KS ? k_slot1 : k_slot0;
        bf16x8 kf[8 * kKB];
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
            kf[c * kKB + kb] = lds_read16(Kt + ka[c] + kb * 32 * kRowBytes);
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
#pragma unroll
          for (int kb = 0; kb < kKB; ++kb)
            s[kb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c * kKB + kb], qf[c], s[kb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, kAheadK, 0);
#pragma unroll
        for (int i = 0; i < 8 * kKB - kAheadK; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSgMfma, kAheadK, 0);
      }
    };

    // Softmax phase of tile jj: running max/sum update and P = exp2(...) as bf16.
    auto softmax = [&](int jj) {
      if (jj < 0 || jj >= nT) return;
      if ((t0 + jj + 1) * kBN > lim_lo) {   // keys past this row's limit (last tiles only)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = (t0 + jj) * kBN + kb * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
            if (key >= lim_row) s[kb][v] = -INFINITY;
          }
      }
      // P = 2^(s c - m) and its per-lane partial sums
      float sg[4];
      auto exps = [&]() __attribute__((always_inline)) {
        const float neg_m = -m_used;
#pragma unroll
        for (int kc = 0; kc < kKC; ++kc) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(fmaf(s[kc >> 1][8 * (kc & 1) + e], a.scale_log2, neg_m));
            // each partial sum starts at its first weight (no addition to 0)
            if (kc == 0 && e < 4) sg[e] = p[e];
            else sg[e & 3] += p[e];
          }
          f32x8 pv = {p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]};
          pf[kc] = __builtin_convertvector(pv, bf16x8);
        }
      };
      // The range's first tile forms the row maxima. On a later tile a row whose
      // maximum is still -inf would get weights of inf or NaN, which the sum
      // check below sends through the exact path as well.
      bool exact = jj == 0;
      if (!exact) {
        exps();
        const float big = fmaxf(fmaxf(sg[0], sg[1]), fmaxf(sg[2], sg[3]));
        exact = __any(!(big <= kSumLimit));
      }
      if (exact) {
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int v = 2; v < 16; ++v) mx = fmaxf(mx, s[0][v]);
#pragma unroll
        for (int kb = 1; kb < kKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                           false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float mt = mx * a.scale_log2;
        if (__any(mt > m_used + kRescaleThreshold)) {
          const float mn = fmaxf(m_used, mt);
          // a row with no visible key yet keeps m = -inf (and alpha 1, not NaN)
          const float alpha = mn == m_used ? 1.0f : __builtin_amdgcn_exp2f(m_used - mn);
#pragma unroll
          for (int i = 0; i < 4; ++i) ls[i] *= alpha;
#pragma unroll
          for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int v = 0; v < 16; ++v) oacc[d][v] *= alpha;
          m_used = mn;
        }
        exps();
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) ls[i] += sg[i];
    };

    // Two groups of waves run the same phase sequence, group 1 one interval
    // behind group 0, so that in every interval one wave of each SIMD is in a
    // GEMM phase (MFMA) while the other is in a softmax phase (VALU):
    //   phase 2j: GEMM(j) = PV(j-1) + S(j);   phase 2j+1: softmax(j).
    // Tile j's K and tile j-1's V stay in LDS for intervals 2j and 2j+1; the
    // slots of K(j-1) and V(j-2) are free from interval 2j on (their last
    // reader, group 1's GEMM(j-1), ran in interval 2j-1). Group 1 loads K(j+1)
    // during its softmax phase of interval 2j and waits for it at the end of
    // its GEMM phase of interval 2j+1; group 0 loads V(j) during its softmax
    // phase of interval 2j+1 and waits for it at the end of that phase. Both
    // waits come before the barrier that publishes the tiles, in place for
    // group 0's GEMM(j+1) in interval 2j+2.
    const int nIntervals = 2 * nT + 2;
    for (int i = 0; i < nIntervals; i += 4) {
      const int j0 = i >> 1;
      if (group == 0) gemm(Int<0>{}, j0);
      else {
        if (j0 + 1 < nT) dma_k(j0 + 1, Int<1>{});
        softmax(j0 - 1);
      }
      phase_barrier();
      if (group == 0) {
        if (j0 < nT) dma_v(j0, Int<0>{});
        softmax(j0);
      } else gemm(Int<0>{}, j0);
      __builtin_amdgcn_s_waitcnt(kWaitLoads);
      phase_barrier();
      const int j1 = j0 + 1;
      if (group == 0) gemm(Int<1>{}, j1);
      else {
        if (j1 + 1 < nT) dma_k(j1 + 1, Int<0>{});
        softmax(j0);
      }
      phase_barrier();
      if (group == 0) {
        if (j1 < nT) dma_v(j1, Int<1>{});
        softmax(j1);
      } else gemm(Int<1>{}, j1);
      __builtin_amdgcn_s_waitcnt(kWaitLoads);
      phase_barrier();
    }

    // ---- epilogue: combine the two half-waves' partial sums, normalise, store.
    float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                       false, false);
      lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (split >= 0) {
      // partial result of this key range: O unnormalised (relative to m),
      // then m and l per row; rows past Lq are written too and never read
      float* pp = a.part + (int64_t)split * kAttnPartFloats;
      const int prow = wave * 32 + r32;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          *reinterpret_cast<f32x4*>(pp + prow * kHD + 32 * db + 8 * a4 + 4 * hf) =
              f32x4{oacc[db][4 * a4], oacc[db][4 * a4 + 1], oacc[db][4 * a4 + 2],
                    oacc[db][4 * a4 + 3]};
      if (hf == 0) {
        pp[kBM * kHD + prow] = m_used;
        pp[kBM * kHD + kBM + prow] = lsum;
      }
    } else {
      // Normalised bf16 rows go through LDS (every K/V slot is free after the
      // loop's last barrier): each wave stages its own 32 x 128 block, 16-byte
      // chunk c of row r at chunk c ^ (r % 16), then stores whole 256-byte row
      // segments, 4 rows per instruction, instead of 16-byte pieces of 32 rows.
      const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
      char* const st = ((wave >> 1) == 0 ? k_slot0 : (wave >> 1) == 1 ? k_slot1
                        : (wave >> 1) == 2 ? v_slot0 : v_slot1) + (wave & 1) * (32 * kRowBytes);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          f32x4 x = {oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv,
                     oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv};
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const bf16x4 y = __builtin_convertvector(x, bf16x4);
          *reinterpret_cast<u32x2*>(st + r32 * kRowBytes + (((4 * db + a4) ^ (r32 & 15)) << 4) + 8 * hf) =
              __builtin_bit_cast(u32x2, y);
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes done
      const int rq = lane >> 4, ch = lane & 15;
      uint16_t* const obase = static_cast<uint16_t*>(a.o) + h * kHD + 8 * ch;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + rq;
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + r * kRowBytes + ((ch ^ (r & 15)) << 4));
        const int row = qt * kBM + wave * 32 + r;
        if (row < a.Lq) *reinterpret_cast<u32x4*>(obase + ((int64_t)b * a.Lq + row) * a.ld_o) = v;
      }
      if (qrow < a.Lq && a.lse && hf == 0) {
        a.lse[((int64_t)b * a.H + h) * a.Lq + qrow] =
            lsum > 0.f ? m_used * 0.6931471805599453f + logf(lsum) : -INFINITY;
      }
    }
    if (kKind != 1) break;
    item += gridDim.x;
    if (item >= total) break;
    __syncthreads();   // the next item reuses the LDS slots
  }
}

// Combines the key-split partial results of the last work items: for query
// row i with ranges s, M = max_s m_s, w_s = 2^(m_s - M), o_i = sum_s w_s O_s /
// sum_s w_s l_s and lse = M ln 2 + ln(sum_s w_s l_s) (no visible key: o = 0,
// lse = -inf). One thread per (row, 4 channels), 8 rows per block.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int nQ = (a.Lq + kBM - 1) / kBM;
  const int64_t t = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);   // tail row
  const int c4 = threadIdx.x & 31;                                   // channels 4 c4 .. +3
  const int tail_item = (int)(t / kBM), prow = (int)(t % kBM);
  const uint32_t logical = a.n_full + tail_item;
  const int qt = logical % nQ, bh = logical / nQ, h = bh % a.H, b = bh / a.H;
  const int qrow = qt * kBM + prow;
  if (qrow >= a.Lq) return;
  const float* base = a.part + (int64_t)tail_item * a.n_split * kAttnPartFloats;
  float M = -INFINITY;
  for (int sp = 0; sp < a.n_split; ++sp)
    M = fmaxf(M, base[sp * kAttnPartFloats + kBM * kHD + prow]);
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < a.n_split; ++sp) {
    const float* pp = base + sp * kAttnPartFloats;
    const float ms = pp[kBM * kHD + prow];
    if (ms == -INFINITY) continue;   // no visible key in this range
    const float w = __builtin_amdgcn_exp2f(ms - M);
    l += w * pp[kBM * kHD + kBM + prow];
    const f32x4 os = *reinterpret_cast<const f32x4*>(pp + prow * kHD + 4 * c4);
    acc += w * os;
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 y = __builtin_convertvector(acc * inv, bf16x4);
  uint16_t* orow = static_cast<uint16_t*>(a.o) + ((int64_t)b * a.Lq + qrow) * a.ld_o + h * kHD;
  *reinterpret_cast<u32x2*>(orow + 4 * c4) = __builtin_bit_cast(u32x2, y);
  if (a.lse && c4 == 0)
    a.lse[((int64_t)b * a.H + h) * a.Lq + qrow] =
        l > 0.f ? M * 0.6931471805599453f + logf(l) : -INFINITY;
}

hipError_t launch_attn_fwd(const AttnArgs& a, int kind, hipStream_t s) {
  const int nQ = (a.Lq + kBM - 1) / kBM;
  const int64_t total = (int64_t)a.B * a.H * nQ;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)total), block(kThreads);
  switch (kind) {
    case 0:
      if (a.part) {
        const int64_t tail = total - a.n_full;
        if (tail <= 0 || a.n_split < 2) return hipErrorInvalidValue;
        hipLaunchKernelGGL(attn_fwd_kernel<0>, dim3((unsigned)(a.n_full + tail * a.n_split)), block,
                           0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)(tail * kBM / 8)), dim3(256), 0, s, a);
      } else {
        hipLaunchKernelGGL(attn_fwd_kernel<0>, grid, block, 0, s, a);
      }
      break;
    case 1:
      hipLaunchKernelGGL(attn_fwd_kernel<1>, dim3((unsigned)(total < 256 ? total : 256)), block, 0,
                         s, a);
      break;
    case 2: hipLaunchKernelGGL(attn_fwd_kernel<2>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_device_mutex;
int g_cus[kMaxDevices];                 // 0: not looked up yet
void* g_scratch[kMaxDevices];           // device address of `scratch`; nullptr: not looked up yet
constexpr uint64_t kScratchBytes = 256 * kAttnPartFloats * 4;

}  // namespace

// Key-split partial results of the allocation-free entry point: one partial
// per compute unit of a 256-unit device (34 MB, held by each GPU the library
// runs on until the process ends).
static __device__ __align__(256) char scratch[kScratchBytes];

hipError_t device_scratch(void** p, uint64_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_device_mutex);
  if (g_scratch[dev] == nullptr) {
    // In host code `scratch` is only a stand-in: the device address of this
    // device's copy comes from the runtime, looked up once per device with
    // that device current.
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = ptr;
  }
  *p = g_scratch[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

hipError_t device_cu_count(int* n) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_device_mutex);
  if (g_cus[dev] == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_cus[dev] = cus;
  }
  *n = g_cus[dev];
  return hipSuccess;
}

}  // namespace wan
