// Absorbed-MLA attention over the selected latent rows (stage 3 of the LSA hot path).
//
// For each query row and head: logits l_s = scale * q . kv[s, :Dqk] over the selected rows s,
// softmax, and out = sum_s p_s kv[s, :Dv]  (page "MLX-VLM 的 LongCat-Flash-Lite-Sparse ...",
// section "LSA": decode gathers the latent rows named by the top-k indices, prefill applies
// the same selection as a sparse mask; section "架构总览": kv_lora_rank 512 and rope 64, so a
// row is 576 values and the value vector is its first 512).  Decode and prefill share this
// kernel: a prefill chunk is B*Lq independent query rows, each with its own selection.
//
// Design for gfx950.  A workgroup owns one (query row, group of 32 heads, slice of the selected
// rows) and runs four wavefronts; its LDS stays under 80 KB so that two workgroups share a CU
// and hide each other's latency (prefill rows; decode splits are sized for about one per CU).
// The slice is cut into 16-row tiles that stream through a 3-stage LDS ring filled by LDS-DMA
// loads (global_load_lds_dwordx4: a lane names one 16-byte piece of a latent row and the
// hardware writes it straight into LDS), so one to two tiles are in flight while one is
// computed, without holding any of it in registers.  Every 1152-byte
// row is read whole by consecutive lanes.  Within LDS, each tile row permutes its 16-byte units
// by an XOR swizzle chosen for the two read patterns below.
//  * logits: S (32 heads x 16 rows) = Q . KV_tile^T on the 16x16x32 bf16 matrix core, the
//    Dqk/32 steps split over the four wavefronts (each keeps its steps' query fragments in
//    registers).  The four fp32 partial sums are exchanged through LDS and added in a fixed
//    order; each lane reads back exactly the 8 logits (one head, 8 rows) it needs as the A
//    operand of the value product, so every wavefront holds the same logits.
//  * online softmax in fp32, computed identically by every wavefront: base-2 exponentials
//    (log2(e) folded into the scale), one permlane swap per reduction; the running sum adds
//    the bf16-rounded probabilities, so the normalisation matches what the value product sees.
//    The reference maximum moves only when a head's maximum exceeds it by more than 2^8 (the
//    result is the same for any reference; this only bounds the exponentials), so the output
//    accumulators are normally never rescaled.
//  * values: each wavefront accumulates O (32 heads x Dv/4 columns) += P . V with the 32x32x16
//    matrix core (K = the tile's 16 rows); each B operand (8 rows of one column per lane) comes
//    from two LDS transpose reads (ds_read_b64_tr_b16).
//  * several workgroups per query row (decode with few rows) each write their normalised
//    partial output in bf16 (half the bytes of fp32: this traffic is written back to HBM
//    behind later kernels) with its fp32 (max, sum); a combine kernel merges them with
//    log-sum-exp weights in fp32.
#include <algorithm>
#include <type_traits>

#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kThreads = 256;     // 4 wavefronts
constexpr int kTile = 16;         // latent rows per tile
constexpr int kStages = 3;        // LDS ring depth
constexpr int kHeadGroup = 32;    // heads per workgroup
constexpr int kMaxSplits = 64;    // one per lane in the combine
constexpr int kMaxRowsPerSplit = 2048;  // row positions of a split staged in LDS
constexpr int kPartStride = 20;   // floats per head in the partial-logit exchange (16 rows + pad)
constexpr int kTargetWorkgroups = 256;  // one per CU (see make_plan)
constexpr int kMinKeysPerSplit = 64;    // four tiles
constexpr int kCombineThreads = 256;   // four (row, head) pairs per workgroup
constexpr int kXcds = 8;               // accelerator complex dies (one L2 each)
constexpr float kRescaleSlack = 8.0f;   // log2 units the running max may exceed the reference
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int DQK, int DV>
struct Cfg {
  static constexpr int UNITS = DQK / 8;                  // 16-byte units per latent row
  static constexpr int KS = (DQK + 31) / 32;             // 16x16x32 steps over Dqk
  static constexpr int KSW = (KS + 3) / 4;               // steps per wavefront (max)
  static constexpr int NB = DV / 32;                     // 32-column output blocks
  static constexpr int NBW = (NB + 3) / 4;               // blocks per wavefront (max)
  static constexpr int TILE_UNITS = kTile * UNITS;
  static constexpr int NI = (TILE_UNITS + kWave - 1) / kWave;  // DMA instructions per tile
  static constexpr int DPW = (NI + 3) / 4;               // ... per wavefront
  static constexpr int STAGE_UNITS = 4 * DPW * kWave;    // tile plus padding pieces
  static_assert(DQK % 8 == 0 && DV % 32 == 0 && DV <= DQK, "unsupported head dims");
  // Tile row r permutes its 16-byte units inside each aligned group of eight by XOR with
  // swz(r), a GF(2)-linear function of the row's bits 1..3; units past the last full group stay
  // in place.  Among all such masks and all rotations by a multiple of r, this one was measured
  // fastest for the two read patterns of the loop together (16-byte reads of one unit column
  // over the 16 rows, and 8-byte transpose reads of 8 rows x 4 units).
  static constexpr int SWZ_UNITS = UNITS & ~7;
  __device__ static constexpr int swz(int r) {
    return ((r & 2) ? 7 : 0) ^ ((r & 4) ? 4 : 0) ^ ((r & 8) ? 5 : 0);
  }
  // LDS unit holding logical unit c (< UNITS) of tile row r
  __device__ static constexpr int slot(int r, int c) {
    return r * UNITS + (c < SWZ_UNITS ? c ^ swz(r) : c);
  }
  // logical unit stored at LDS unit u (< UNITS) of row r (the permutation is an involution)
  __device__ static constexpr int logical(int r, int u) {
    return u < SWZ_UNITS ? u ^ swz(r) : u;
  }
};

struct MlaParams {
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* indices;
  const int32_t* n_sel;
  const int32_t* seqlens;
  // positions appended after the index pass (multi-token-prediction draft steps): with
  // index_seqlens, row (b, i) also attends to [index_seqlens[b], p], at most max_app of them
  const int32_t* index_seqlens;
  int max_app;
  int Lq, H, S_max, topk;
  int rows;                  // query rows (B * Lq)
  int hgroups, splits, kps;  // head groups, workgroups per (row, head group), rows per split
  int pairs;                 // query rows x heads
  float scale_log2;
  uint16_t* out;
  float* lse;
  uint16_t* ws_o;  // [rows][hgroups][splits][32][DV] normalised partial outputs (bf16)
  float* ws_ml;  // [rows][hgroups][splits][32][2]  reference max (base 2) and sum
};

// One LDS-DMA load: each lane's 16 bytes at `src` land at LDS byte address
// lds_base + 16 * lane.  It is issued from inline assembly on purpose: the compiler's waitcnt
// pass would otherwise treat every later LDS transpose read as possibly aliasing an unfinished
// DMA and drain the whole ring (vmcnt(0)) before it.  This kernel tracks the ring itself with
// explicit vmcnt waits and barriers.  The LDS destination goes in M0 as an input operand bound
// to that register, so the compiler itself writes M0 and knows what it holds.  The instruction
// has no destination registers.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_base) : "memory");
}

// Workgroup barrier for the DMA ring.  __syncthreads() also releases this wavefront's pending
// global->LDS DMA writes, i.e. waits for vmcnt(0), which would drain the ring every step.  Here
// the caller has already waited for exactly the DMA loads the next phase reads (wait_vmcnt<N>),
// so only this wavefront's own LDS accesses are drained before the hardware barrier.  The empty
// asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// D = A * B + C on the 16x16x32 bf16 matrix core.  Per lane l (c = l % 16, q = l / 16):
//   A: row c, k = 8q .. 8q+7;  B: column c, k = 8q .. 8q+7;  C/D register r: row 4q + r, column c.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// SPARSE: the rows come from P.indices (else every position 0..p, the dense fallback).
template <int DQK, int DV, bool SPARSE>
__global__ __launch_bounds__(kThreads, 2) void sparse_mla_kernel(MlaParams P) {
  using C = Cfg<DQK, DV>;
  // One LDS block in a fixed order: the row-position slice, read every tile, sits at the bottom,
  // so that every LDS offset of the loop fits an instruction's 16-bit immediate.
  struct Smem {
    int32_t slice[kMaxRowsPerSplit];
    __attribute__((aligned(16))) float spart[4][kHeadGroup * kPartStride];  // partial logits
    __attribute__((aligned(16))) float inv_head[kHeadGroup];  // 1 / l per head (epilogue)
    __attribute__((aligned(1024))) uint16_t ring[kStages][C::STAGE_UNITS * 8];
  };
  __shared__ __attribute__((aligned(1024))) Smem sm;
  auto& slice = sm.slice;
  auto& spart = sm.spart;
  auto& inv_head = sm.inv_head;
  auto& ring = sm.ring;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int col = lane & 31, g = lane >> 5;   // 32x32 layouts
  const int c16 = lane & 15, q16 = lane >> 4;  // 16x16 layouts
  // XCD-aware work order: the dispatcher deals workgroup ids to the 8 XCDs in turn, so id b
  // runs on XCD b % 8.  XCD x takes a contiguous run of (row, head group) units with all their
  // splits: a unit's query is then fetched into one L2, and neighbouring prefill rows, whose
  // selections share the sink and window rows, gather through the same L2.  Units past the
  // last multiple of 8 keep the plain order.
  const int bid = blockIdx.x;
  const int units = P.rows * P.hgroups;
  const int per_xcd = units / kXcds;  // units per XCD in the XCD-aware part
  int unit, split;
  if (bid < per_xcd * kXcds * P.splits) {
    const int l = bid / kXcds;
    unit = (bid % kXcds) * per_xcd + l / P.splits;
    split = l % P.splits;
  } else {
    const int r = bid - per_xcd * kXcds * P.splits;
    unit = per_xcd * kXcds + r / P.splits;
    split = r % P.splits;
  }
  const int hg = unit % P.hgroups;
  const int row = unit / P.hgroups;
  const int b = row / P.Lq;
  const int n = min(P.seqlens[b] - P.Lq + (row - b * P.Lq) + 1, P.S_max);
  constexpr bool sparse = SPARSE;
  const int cnt_sel = sparse ? min(P.n_sel[row], P.topk) : max(n, 0);
  int cnt = cnt_sel, app0 = 0;
  if (sparse && P.index_seqlens) {
    app0 = max(P.index_seqlens[b], 0);
    cnt += min(max(n - app0, 0), P.max_app);
  }
  const int j0 = split * P.kps;
  // the last split also takes the appended positions (without them cnt <= splits * kps)
  const int j1 = split == P.splits - 1 ? cnt : min(cnt, j0 + P.kps);
  const int ntiles = j1 > j0 ? (j1 - j0 + kTile - 1) / kTile : 0;
  const uint16_t* kv_b = P.kv + static_cast<size_t>(b) * P.S_max * DQK;

  // query fragments of this wavefront's Dqk steps (B operand: column = head, k = dims); they
  // do not depend on the selection, so they are requested first
  bf16x8 qf[2][C::KSW];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = hg * kHeadGroup + 16 * hb + c16;
#pragma unroll
    for (int i = 0; i < C::KSW; ++i) {
      const int ks = wave + 4 * i;
      const int dim0 = 32 * ks + 8 * q16;
      qf[hb][i] = (head < P.H && ks < C::KS && dim0 < DQK)
                      ? load_bf16x8(P.q + (static_cast<size_t>(row) * P.H + head) * DQK + dim0)
                      : zero_bf16x8();
    }
  }
  // this split's row positions (clamped into the cache) staged in LDS, padded to whole tiles
  // with the last one (rows past the slice repeat its last row), so a tile's lookups need no
  // clamp
  if constexpr (sparse) {
    const int32_t* ilist = P.indices + static_cast<size_t>(row) * P.topk;
    for (int j = tid; j < ntiles * kTile; j += kThreads) {
      const int jj = j0 + min(j, j1 - j0 - 1);
      slice[j] = jj < cnt_sel ? min(max(ilist[jj], 0), P.S_max - 1) : app0 + (jj - cnt_sel);
    }
  }
  // retire the query and index loads here: a wait left to the compiler would sit inside the
  // loop and drain the ring on every step
  wait_vmcnt<0>();
  __syncthreads();

  // DMA pieces of this wavefront: instruction k covers tile units (4k + wave) * 64 + lane
  int dma_r[C::DPW], dma_c[C::DPW];
#pragma unroll
  for (int k = 0; k < C::DPW; ++k) {
    const int u = (4 * k + wave) * kWave + lane;
    const bool real = u < C::TILE_UNITS;  // padding pieces re-read row 0, unit 0
    const int r = real ? u / C::UNITS : 0;
    dma_r[k] = r;
    dma_c[k] = real ? C::logical(r, u - r * C::UNITS) : 0;
  }
  // cache row positions of the next tile to be issued, read from LDS one step ahead so that
  // the issue itself waits on nothing
  int pos[C::DPW];
  auto fetch_pos = [&](int tile) {  // tile < ntiles
    const int jb = tile * kTile;  // relative to j0
#pragma unroll
    for (int k = 0; k < C::DPW; ++k) {
      if constexpr (sparse) pos[k] = slice[jb + dma_r[k]];
      else pos[k] = j0 + min(jb + dma_r[k], j1 - j0 - 1);  // past the end: the last row again
    }
  };
  auto issue = [&](uint16_t* stage) {
#pragma unroll
    for (int k = 0; k < C::DPW; ++k) {
      const uint16_t* src = kv_b + static_cast<size_t>(pos[k]) * DQK + 8 * dma_c[k];
      dma16(src, static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                     (lds_void*)(stage + (4 * k + wave) * kWave * 8))));
    }
  };
  if (ntiles > 0) {
    fetch_pos(0);
    issue(ring[0]);
    if (ntiles > 1) {
      fetch_pos(1);
      issue(ring[1]);
    }
    if (ntiles > 2) fetch_pos(2);
  }

  // LDS element offsets of this lane's fragment reads within a stage.  Keys: step i reads
  // logical unit c0 + 16 i of tile row c16; the swizzle only permutes units inside groups of
  // eight, so steps before the last sit at k_lane + 128 i, and the last step, which may lie past
  // Dqk (it then meets a zero query fragment), reads a clamped in-row unit.  Values: column
  // block wave + 4 i starts at unit 4 (wave + 4 i), i.e. at v_lane + 128 i, for transpose-read
  // row group h2 (rows 8 h2 + 4 (G >> 1) + (jl >> 2), 4 columns per lane group).
  static_assert(C::KSW == 1 || 16 * (C::KSW - 1) <= C::SWZ_UNITS, "key steps before the last are swizzled");
  static_assert(C::NBW == 1 || DV / 8 <= C::SWZ_UNITS, "value units are swizzled");
  const int c0 = 4 * wave + q16;
  const int k_lane = C::slot(c16, min(c0, C::UNITS - 1)) * 8;
  const int k_last = C::slot(c16, min(c0 + 16 * (C::KSW - 1), C::UNITS - 1)) * 8;
  int v_lane[2];
  {
    const int G = lane >> 4, jl = lane & 15;
    const int dim0 = 32 * wave + 16 * (G & 1) + 4 * (jl & 3);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int vr = 8 * h2 + 4 * (G >> 1) + (jl >> 2);  // = acc_row(4*h2 + k, g) for slot k
      v_lane[h2] = C::slot(vr, min(dim0 >> 3, C::UNITS - 1)) * 8 + (dim0 & 7);
    }
  }

  float m_ref = -INFINITY, l_run = 0.0f;  // for head `col` (identical in every wavefront)
  f32x16 o[C::NBW];
#pragma unroll
  for (int i = 0; i < C::NBW; ++i) o[i] = f32x16{};

  // Tile t, in ring stage S = t % kStages.  The loop below is unrolled by kStages so that S is
  // a compile-time constant: every LDS address is then a per-lane register plus an immediate.
  auto tile_step = [&](const int t, auto stage) {
    constexpr int S = decltype(stage)::value;
    if (t + 1 < ntiles) wait_vmcnt<C::DPW>();  // tile t+1 may still be in flight
    else wait_vmcnt<0>();
    ring_barrier();  // every wavefront's pieces of tile t are in LDS; tile t - 1 is consumed
    // tile t + 2 goes into the stage of tile t - 1: every wavefront has passed the barrier
    // above, so all of its reads of that stage (and of the partial logits) are complete
    if (t + 2 < ntiles) {
      issue(ring[(S + 2) % kStages]);
      if (t + 3 < ntiles) fetch_pos(t + 3);
    }

    const uint16_t* kvt = ring[S];
    // ---- partial logits over this wavefront's Dqk steps, as S^T = KV_tile . Q^T so that a
    // lane holds one head (c16) for four consecutive tile rows (4*q16 + r): one 16-byte LDS
    // write per head block
    {
      // every wavefront runs KSW steps: a step past Dqk reads an in-range unit (finite cache
      // values) against the zero query fragment loaded for it, so it adds exactly 0
      f32x4 acc0 = {}, acc1 = {};
      bf16x8 kb[C::KSW];
#pragma unroll
      for (int i = 0; i < C::KSW; ++i)
        kb[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                               kvt + (i + 1 < C::KSW ? k_lane + 128 * i : k_last)));
      __builtin_amdgcn_sched_barrier(0);  // every fragment read is issued before the first step
#pragma unroll
      for (int i = 0; i < C::KSW; ++i) {
        acc0 = mfma16(kb[i], qf[0][i], acc0);
        acc1 = mfma16(kb[i], qf[1][i], acc1);
      }
      float* sp = spart[wave];
      *reinterpret_cast<f32x4*>(&sp[c16 * kPartStride + 4 * q16]) = acc0;
      *reinterpret_cast<f32x4*>(&sp[(16 + c16) * kPartStride + 4 * q16]) = acc1;
    }
    ring_barrier();  // partial logits of all wavefronts published

    // ---- logits of head `col` for the tile rows of A-operand slots e: acc_row(e, g)
    float sv[8];
    {
      f32x4 lw[4], hw[4];  // all eight reads are issued before the first add
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float* pw = &spart[w][col * kPartStride + 4 * g];
        lw[w] = *reinterpret_cast<const f32x4*>(pw);
        hw[w] = *reinterpret_cast<const f32x4*>(pw + 8);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4 lo = lw[0], hi = hw[0];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        lo += lw[w];
        hi += hw[w];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[e] = lo[e];
        sv[4 + e] = hi[e];
      }
    }

    // ---- value-operand fragments of this wavefront's 32-column blocks: they do not depend on
    // the probabilities, so they are requested here and arrive during the softmax.  Each B
    // operand (8 tile rows of one column per lane) is two LDS transpose reads.
    u32x2 hv[C::NBW][2];
#pragma unroll
    for (int i = 0; i < C::NBW; ++i) {
      if (C::NB % 4 == 0 || wave + 4 * i < C::NB) {  // statically true when the blocks divide evenly
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
          hv[i][h2] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(kvt + v_lane[h2] + 128 * i)));
      }
    }

    // ---- online softmax for head `col` (every wavefront computes the same values)
    const int tile_j = j0 + t * kTile;
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] *= P.scale_log2;
    if (tile_j + kTile > j1) {  // the slice's last, partial tile: rows past its end drop out
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (tile_j + acc_row(e, g) >= j1) sv[e] = -INFINITY;
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) mloc = fmaxf(mloc, sv[e]);
    mloc = max_xor32(mloc);
    const bool grow = mloc > m_ref + kRescaleSlack;
    if (__ballot(grow)) {
      const float m_new = grow ? mloc : m_ref;
      const float alpha = exp2f(m_ref - m_new);  // 0 while nothing has been accumulated
      l_run *= alpha;
      m_ref = m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float a = __shfl(alpha, acc_row(r, g));  // heads of O held by this lane
#pragma unroll
        for (int i = 0; i < C::NBW; ++i) o[i][r] *= a;
      }
    }
    // probabilities: the hardware exponential (results below 2^-126 of the reference flush to
    // zero; every row's largest probability is at least 2^-8) and the paired round-to-nearest-
    // even conversion to bf16
    uint32_t pw[4];
    float psum = 0.0f;
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 pr = {static_cast<__bf16>(__builtin_amdgcn_exp2f(sv[2 * i] - m_ref)),
                         static_cast<__bf16>(__builtin_amdgcn_exp2f(sv[2 * i + 1] - m_ref))};
      pw[i] = __builtin_bit_cast(uint32_t, pr);
      psum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, psum, false);  // both bf16 values, in fp32
    }
    psum = sum_xor32(psum);
    l_run += psum;
    // A operand: k-slot e of lane half g is tile row acc_row(e, g)
    const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});

    // ---- values: O (32 heads x this wavefront's blocks nb = wave + 4i) += P . V_tile
#pragma unroll
    for (int i = 0; i < C::NBW; ++i) {
      const int nb = wave + 4 * i;
      if (C::NB % 4 == 0 || nb < C::NB)
        o[i] = mfma32(pa, __builtin_bit_cast(bf16x8, u32x4{hv[i][0].x, hv[i][0].y, hv[i][1].x, hv[i][1].y}),
                      o[i]);
    }
  };
  static_assert(kStages == 3, "the tile loop is unrolled by the ring depth");
  for (int t = 0; t < ntiles; t += kStages) {
    tile_step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) tile_step(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < ntiles) tile_step(t + 2, std::integral_constant<int, 2>{});
  }
  wait_vmcnt<0>();
  if (wave == 0 && g == 0) inv_head[col] = l_run > 0.0f ? 1.0f / l_run : 0.0f;
  __syncthreads();  // the epilogue below reuses the ring: every wavefront's last reads are done

  // ---- epilogue: normalise, round to bf16 and stage this workgroup's [32 heads x DV] block in
  // LDS (the ring is free now), then write it out with 16-byte nontemporal stores (read once, by
  // the combine): rows of the output for one split, or this head group's rows of `out` when
  // there is a single split
  {
    uint16_t* tb = &ring[0][0];
    static_assert(kStages * C::STAGE_UNITS * 8 >= kHeadGroup * DV, "the ring holds the block");
    // 1 / l of the heads this lane holds: rows acc_row(r, g) = 8 (r / 4) + 4 g + r % 4
    f32x4 inv4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) inv4[q] = *reinterpret_cast<const f32x4*>(&inv_head[8 * q + 4 * g]);
    // adjacent columns live in lanes col and col ^ 1: one DPP swap per row pair lets the even
    // lane write row r's columns (col, col + 1) and the odd lane row r + 1's (col - 1, col) as
    // one 4-byte store each
    const bool odd = (col & 1) != 0;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int hrow = acc_row(r, g) + (odd ? 1 : 0);  // acc_row(r + 1, g) = acc_row(r, g) + 1
      const float i0 = inv4[r >> 2][r & 3], i1 = inv4[r >> 2][(r & 3) + 1];
#pragma unroll
      for (int i = 0; i < C::NBW; ++i) {
        const int nb = wave + 4 * i;
        if (C::NB % 4 == 0 || nb < C::NB) {
          const float v0 = o[i][r] * i0, v1 = o[i][r + 1] * i1;
          const float got = __int_as_float(__builtin_amdgcn_update_dpp(
              0, __float_as_int(odd ? v0 : v1), 0xB1, 0xf, 0xf, false));  // quad_perm [1,0,3,2]
          const bf16x2 pr = odd ? bf16x2{static_cast<__bf16>(got), static_cast<__bf16>(v1)}
                                : bf16x2{static_cast<__bf16>(v0), static_cast<__bf16>(got)};
          *reinterpret_cast<uint32_t*>(&tb[hrow * DV + 32 * nb + (col & ~1)]) =
              __builtin_bit_cast(uint32_t, pr);
        }
      }
    }
    __syncthreads();
    const bool direct = P.splits == 1;
    const size_t slot = (static_cast<size_t>(row) * P.hgroups + hg) * P.splits + split;
    uint16_t* dst = direct ? P.out + (static_cast<size_t>(row) * P.H + hg * kHeadGroup) * DV
                           : P.ws_o + slot * kHeadGroup * DV;
    const int rows_out = direct ? min(kHeadGroup, P.H - hg * kHeadGroup) : kHeadGroup;
    const int n_out = rows_out * DV;  // elements of the block that exist in the destination
    if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0u) {
      for (int e = 8 * tid; e < n_out; e += 8 * kThreads)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(tb + e), reinterpret_cast<u32x4*>(dst + e));
    } else {  // a caller buffer without 16-byte alignment
      for (int e = tid; e < n_out; e += kThreads) dst[e] = tb[e];
    }
    if (direct) {
      const int head = hg * kHeadGroup + col;
      if (wave == 0 && g == 0 && head < P.H && P.lse)
        P.lse[static_cast<size_t>(row) * P.H + head] =
            l_run > 0.0f ? (m_ref + __log2f(l_run)) * kLn2 : -INFINITY;
    } else if (wave == 0 && g == 0) {
      P.ws_ml[(slot * kHeadGroup + col) * 2] = m_ref;
      P.ws_ml[(slot * kHeadGroup + col) * 2 + 1] = l_run;
    }
  }
}

// Merge the split partials of one (row, head) with log-sum-exp weights, in a fixed order: one
// wavefront per (row, head), lane l owning output columns [CPL*l, CPL*l + CPL).  Partial s holds
// O_s / l_s (bf16) and (m_s, l_s); its weight is l_s * 2^(m_s - max).  Lane s reads split s's
// (m, l) and every lane requests its columns of the first 16 splits right behind it, so the
// weights are formed (DPP reductions, no LDS) while the partial outputs are in flight.
template <int DV>
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(MlaParams P) {
  constexpr int CPL = DV / kWave;  // output columns per lane
  static_assert(DV % kWave == 0 && (CPL == 8 || CPL == 1), "combine handles DV = 512 or 64");
  static_assert(kMaxSplits <= kWave && kMaxSplits % 16 == 0, "one split per lane, whole batches");
  using Piece = typename std::conditional<CPL == 8, u32x4, uint32_t>::type;
  constexpr int kBatch = 16;  // partial loads in flight per lane
  const int lane = threadIdx.x & 63;
  const int pair = static_cast<int>(blockIdx.x) * (kCombineThreads / kWave) +
                   __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (pair >= P.pairs) return;  // whole wavefronts
  const int row = pair / P.H, head = pair - row * P.H;
  const int hg = head / kHeadGroup, hl = head - hg * kHeadGroup;
  const int S = P.splits;
  const size_t slot0 = (static_cast<size_t>(row) * P.hgroups + hg) * P.splits;
  const size_t stride = static_cast<size_t>(kHeadGroup) * DV;
  const uint16_t* src = P.ws_o + (slot0 * kHeadGroup + hl) * DV + CPL * lane;
  // (m, l) of split `lane`; lanes past the last split read it too and are given weight 0
  const float2 ml = *reinterpret_cast<const float2*>(
      &P.ws_ml[((slot0 + min(lane, S - 1)) * kHeadGroup + hl) * 2]);
  Piece v[kBatch];
  auto fetch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint16_t* at = src + static_cast<size_t>(min(s0 + u, S - 1)) * stride;
      if constexpr (CPL == 8) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(at));
      else v[u] = *at;
    }
  };
  fetch(0);
  __builtin_amdgcn_sched_barrier(0);  // keep the partial loads ahead of the weights
  const float ms = lane < S ? ml.x : -INFINITY;
  const float mmax = wave_max_f(ms);
  const float wgt = (ms == -INFINITY) ? 0.0f : exp2f(ms - mmax) * ml.y;
  const float L = wave_sum_f(wgt);
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
  for (int s0 = 0;;) {
    // splits past the last (s0 + u >= S < 64) have weight 0 and re-read split S - 1
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), s0 + u));
      if constexpr (CPL == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += w * __uint_as_float(v[u][i] << 16);
          acc[2 * i + 1] += w * __uint_as_float(v[u][i] & 0xffff0000u);
        }
      } else {
        acc[0] += w * __uint_as_float(v[u] << 16);
      }
    }
    s0 += kBatch;
    if (s0 >= S) break;
    fetch(s0);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  uint16_t* dst = P.out + (static_cast<size_t>(row) * P.H + head) * DV + CPL * lane;
  if constexpr (CPL == 8) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = __builtin_bit_cast(uint32_t, bf16x2{static_cast<__bf16>(acc[2 * i] * inv),
                                                 static_cast<__bf16>(acc[2 * i + 1] * inv)});
    if ((reinterpret_cast<uintptr_t>(P.out) & 15u) == 0u) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    } else {  // a caller buffer without 16-byte alignment
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[2 * i] = static_cast<uint16_t>(w[i]);
        dst[2 * i + 1] = static_cast<uint16_t>(w[i] >> 16);
      }
    }
  } else {
    dst[0] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[0] * inv));
  }
  if (lane == 0 && P.lse)
    P.lse[static_cast<size_t>(row) * P.H + head] = L > 0.0f ? (mmax + __log2f(L)) * kLn2 : -INFINITY;
}

struct MlaPlan {
  int hgroups = 1, splits = 1, kps = 0;
  size_t ws_o_bytes = 0, ws_ml_bytes = 0, ws_slack = 0;
};

MlaPlan make_plan(long rows, int H, int Dv, int S_max, int topk, int dense, int app = 0) {
  MlaPlan pl;
  pl.hgroups = (H + kHeadGroup - 1) / kHeadGroup;
  const long keys = dense ? S_max : topk;
  const long units = rows * pl.hgroups;
  // Decode splits: about one workgroup per CU, each streaming at least four tiles.  Two
  // workgroups fit on a CU, but every split pays a prologue of two dependent memory round trips
  // (indices, then rows) and writes a partial that the combine reads back, so fewer, longer
  // splits win: measured per decode call, 16 tiles x 8 splits beat 8 x 16 at 32 rows, 4 x 32
  // beat 2 x 64 at 8 rows, and 4 tiles x 32 splits beat 2 x 64 at 4 rows.
  long splits = units > 0 ? (kTargetWorkgroups + units - 1) / units : 1;
  splits = std::min<long>(splits, (keys + kMinKeysPerSplit - 1) / kMinKeysPerSplit);
  splits = std::min<long>(splits, kMaxSplits);
  if (!dense) splits = std::max<long>(splits, (keys + kMaxRowsPerSplit - 1) / kMaxRowsPerSplit);
  splits = std::max<long>(splits, 1);
  auto per_split = [&](long sp) {
    const long k = ((keys + sp - 1) / sp + kTile - 1) / kTile * kTile;
    return k < kTile ? static_cast<long>(kTile) : k;
  };
  long kps = per_split(splits);
  // the last split also stages the appended positions: keep them within its LDS slice
  while (!dense && app > 0 && kps + app > kMaxRowsPerSplit && splits < kMaxSplits) kps = per_split(++splits);
  splits = (keys + kps - 1) / kps;
  if (splits < 1) splits = 1;
  pl.splits = static_cast<int>(splits);
  pl.kps = static_cast<int>(std::min<long>(kps, 0x7fffffffL));
  if (pl.splits > 1) {
    const size_t slots = static_cast<size_t>(units) * pl.splits;
    pl.ws_o_bytes = (slots * kHeadGroup * Dv * 2 + 255) & ~static_cast<size_t>(255);
    pl.ws_ml_bytes = (slots * kHeadGroup * 2 * 4 + 255) & ~static_cast<size_t>(255);
    pl.ws_slack = kWorkspaceAlign;
  }
  return pl;
}

template <int DQK, int DV>
hipError_t launch_dims(const MlaParams& P, long rows, hipStream_t stream) {
  const long grid = rows * P.hgroups * P.splits;
  if (grid > 0x7fffffffL || rows * P.H > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (P.indices)
    hipLaunchKernelGGL((sparse_mla_kernel<DQK, DV, true>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, stream, P);
  else
    hipLaunchKernelGGL((sparse_mla_kernel<DQK, DV, false>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, stream, P);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || P.splits == 1) return err;
  constexpr int kPairsPerGroup = kCombineThreads / kWave;
  hipLaunchKernelGGL((mla_combine_kernel<DV>),
                     dim3(static_cast<unsigned>((rows * P.H + kPairsPerGroup - 1) / kPairsPerGroup)),
                     dim3(kCombineThreads), 0, stream, P);
  return hipGetLastError();
}

}  // namespace

size_t mla_workspace_bytes(int B, int Lq, int H, int Dv, int S_max, int topk, int dense, int app) {
  const MlaPlan pl = make_plan(static_cast<long>(B) * Lq, H, Dv, S_max, topk, dense, app);
  return pl.ws_o_bytes + pl.ws_ml_bytes + pl.ws_slack;
}

hipError_t launch_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices,
                      const int32_t* n_sel, const int32_t* seqlens, int B, int Lq, int H, int Dqk,
                      int Dv, int S_max, int topk, float softmax_scale, uint16_t* out, float* lse,
                      void* workspace, hipStream_t stream, const int32_t* index_seqlens,
                      int max_app) {
  const long rows = static_cast<long>(B) * Lq;
  const int app = index_seqlens ? max_app : 0;
  const MlaPlan pl = make_plan(rows, H, Dv, S_max, topk, indices == nullptr, app);
  MlaParams P{};
  P.q = q;
  P.kv = kv;
  P.indices = indices;
  P.n_sel = n_sel;
  P.seqlens = seqlens;
  P.index_seqlens = index_seqlens;
  P.max_app = app;
  P.Lq = Lq;
  P.H = H;
  P.S_max = S_max;
  P.topk = topk;
  P.rows = static_cast<int>(rows);
  P.hgroups = pl.hgroups;
  P.splits = pl.splits;
  P.kps = pl.kps;
  P.scale_log2 = softmax_scale * kLog2e;
  P.out = out;
  P.lse = lse;
  P.pairs = static_cast<int>(std::min<long>(rows * H, 0x7fffffffL));
  char* ws = align_workspace(workspace);
  P.ws_o = reinterpret_cast<uint16_t*>(ws);
  P.ws_ml = reinterpret_cast<float*>(ws + pl.ws_o_bytes);
  if (Dqk == 576 && Dv == 512) return launch_dims<576, 512>(P, rows, stream);
  if (Dqk == 80 && Dv == 64) return launch_dims<80, 64>(P, rows, stream);
  return hipErrorInvalidValue;
}

}  // namespace lsa
