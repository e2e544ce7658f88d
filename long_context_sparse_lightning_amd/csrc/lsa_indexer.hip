// Lightning-indexer scores (stage 1 of the LSA hot path).
//
//   scores[b,i,s] = sum_h w[b,i,h] * max(0, q_idx[b,i,h,:] . k_idx[b,s,:])     for s <= p
//
// (page "MLX-VLM 的 LongCat-Flash-Lite-Sparse ...", section "LSA" for the score, section
// "预填充优化" for the ReLU-weighted head sum done in one fused epilogue without a
// [heads x keys] intermediate.)
//
// Design for gfx950.  One wavefront scores 32 keys at a time with the 32x32x16 bf16 matrix
// core: A = the query's index heads (32 rows, zero-padded past Hi), B = 32 keys; Di/16
// instructions cover the head dimension.  The query fragment stays in registers for the
// whole scan, so the only HBM stream is the key cache, read exactly once.  Each lane loads
// one 16-byte piece of a key per instruction; the two lanes holding a key cover its two
// halves, so the dims are assigned to the k index as: lane half g, step c -> dims
// [g*Di/2 + 8c, +8), identically for A and B (any consistent assignment gives the same dot
// product).  The epilogue multiplies each accumulator row (head) by its weight after the
// ReLU, sums the 16 heads a lane holds, and adds the partner lane's 16 heads: scores leave
// the kernel as one fp32 per key and the [heads x keys] tile never touches memory.
// Loads for the next tile are issued before the matrix-core work of the current one, into the
// other of two register buffers (the loop is unrolled by two, so no register copy has to wait
// for a load in flight), and without a condition: a conditional prefetch makes the compiler
// wait for it together with the current tile.  The last one or two tiles are peeled off the
// loop, so no load past the chunk is left in flight when the scan ends.
// Scores are staged in LDS and written with coalesced stores after the scan: a global store in
// the loop would make the next overwrite of its data register wait for the store -- and, since
// loads and stores share one counter, for every prefetch issued before it.
//
// Query-blocked variant (prefill, many query rows per sequence): the per-row scan above reads a
// sequence's keys once per query row, which makes prefill bound by cache bandwidth.  Here a
// workgroup of 8 wavefronts owns 16 consecutive query rows (2 per wavefront, their query
// fragments and weights in registers) and a chunk of keys.  Each 32-key tile is loaded once per
// workgroup into a 4-slot, XOR-swizzled LDS ring (one 16-byte piece per thread, register
// prefetch ahead); every wavefront reads the next tile's key fragments a step ahead and reuses
// each fragment for both of its rows, and each row's epilogue runs next to the other row's
// matrix-core chain, in an instruction order fixed with scheduling barriers.  Key chunk c goes
// to workgroups c, c + nchunks, ..., which the dispatcher places on one XCD when nchunks is a
// multiple of 8, so each XCD's L2 holds one slice of the keys for every query block.  The work
// is then bound by the matrix cores and their LDS operand traffic.
//
// Fused variant (indexer + top-k, the scores never leave the chip): instead of writing its
// staged scores, a workgroup turns them into its chunk's top-k candidate list (a superset of
// the chunk's contribution to the row's top R, see lsa_select.h), and the top-k merge kernel
// finishes the selection from those lists.  Of the two workgroups on a CU one streams first and
// its selection overlaps the other's scan; the last selection on each CU is exposed after the
// key stream, so that code is kept short (no memory waits, no LDS permutes, no bank conflicts).
#include <algorithm>

#include "lsa_select.h"

namespace lsa {
namespace {

constexpr int kThreads = 256;             // 4 wavefronts (the default workgroup)
constexpr int kWideThreads = 512;         // 8 wavefronts: fused launches of few workgroups
constexpr int kWideMaxGrid = 128;         // ... at most this many (one per CU at 136 VGPRs)
constexpr int kTileKeys = 32;             // keys per wavefront step
constexpr int kWgStride = kTileKeys * 4;  // keys per step of a 4-wavefront workgroup
constexpr int kMaxKeysPerWg = 8192;       // LDS score staging: 32 KB
constexpr size_t kFusedBudget = size_t(256) << 20;     // candidate lists of one row group

struct IndexParams {
  const uint16_t* q_idx;
  const float* w;
  const uint16_t* k_idx;
  const int32_t* seqlens;
  int Lq, Hi, S_max;
  int keys_per_wg, chunks_per_row;
  float* scores;  // plain variant
  // fused variant: rows [row0, row0 + gridDim.x / chunks_per_row), candidate lists per chunk
  int row0, topk, init, local, R;
  uint32_t* count;  // [group rows][chunks]
  uint32_t* range;  // [group rows][chunks][2]
  uint2* cand;      // [group rows][chunks][list_stride]
  int list_stride;  // sel::list_capacity(R, keys_per_wg)
};

// THREADS: 256, or 512 for a fused launch too small to fill the chip (each wavefront keeps one
// key tile in flight, so more wavefronts per workgroup stream more bytes per CU).
template <int DI, bool FUSED, int THREADS = kThreads>
__global__ __launch_bounds__(THREADS) void index_scores_kernel(IndexParams P) {
  constexpr int NC = DI / 16;  // matrix-core steps over the head dimension
  constexpr int WG_STRIDE = kTileKeys * (THREADS / 64);  // keys per workgroup step
  constexpr int STAGE_ITEMS = kMaxKeysPerWg / THREADS;   // staged scores per thread (fused)
  const uint16_t* __restrict__ q_idx = P.q_idx;
  const float* __restrict__ w = P.w;
  const uint16_t* __restrict__ k_idx = P.k_idx;
  const int32_t* __restrict__ seqlens = P.seqlens;
  const int Lq = P.Lq, Hi = P.Hi, S_max = P.S_max, keys_per_wg = P.keys_per_wg;
  const int chunks_per_row = P.chunks_per_row;
  const int grow = blockIdx.x / chunks_per_row;  // row within the launch
  const int chunk = blockIdx.x - grow * chunks_per_row;
  const int row = (FUSED ? P.row0 : 0) + grow;
  const int b = row / Lq;
  // keys visible to this query (clamped so a bad seqlens value cannot write past the row)
  const int n = min(seqlens[b] - Lq + (row - b * Lq) + 1, S_max);
  const int start = chunk * keys_per_wg;
  // fused variant: the competing positions [comp_a, comp_z] of this chunk, found before the scan
  // so the selection after it starts without a memory access (since rg.hi <= n - 1, clipping to
  // the chunk equals clipping to [start, end))
  int comp_a = 0, comp_z = -1;
  if constexpr (FUSED) {
    // chunks holding no competing position produce an empty list (and skip the scan)
    const sel::RowGeom rg = sel::row_geom(seqlens, row, Lq, S_max, P.topk, P.init, P.local);
    comp_a = max(rg.lo, start);
    comp_z = min(rg.hi, start + keys_per_wg - 1);
    if (rg.dense || P.R == 0 || comp_z < comp_a) {
      if (threadIdx.x == 0) P.count[blockIdx.x] = 0u;
      return;
    }
  }
  if (start >= n) return;
  const int end = min(n, start + keys_per_wg);

  const int lane = threadIdx.x & 63;
  // wave index made provably uniform, so the tile loop below is scalar control flow (a
  // divergent loop exit would add a path on which the compiler waits for every load in flight)
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int col = lane & 31;
  const int g = lane >> 5;

  bf16x8 qa[NC];
  {
    const uint16_t* qp = q_idx + (static_cast<size_t>(row) * Hi + col) * DI + g * (DI / 2);
#pragma unroll
    for (int c = 0; c < NC; ++c) qa[c] = col < Hi ? load_bf16x8(qp + 8 * c) : zero_bf16x8();
  }
  float wr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int h = acc_row(r, g);
    wr[r] = h < Hi ? w[static_cast<size_t>(row) * Hi + h] : 0.0f;
  }
  extern __shared__ __attribute__((aligned(16))) float stage[];  // [keys_per_wg] scores of this chunk
  // fused variant: the selection's histogram (2 * kBins words) follows the scores and is cleared
  // now, while the query loads are in flight, so the selection after the scan starts with it
  uint32_t* hist = reinterpret_cast<uint32_t*>(stage + keys_per_wg);  // keys_per_wg % 128 == 0
  if constexpr (FUSED)
    for (int i = threadIdx.x; i < 2 * sel::kBins / 4; i += THREADS)
      reinterpret_cast<u32x4*>(hist)[i] = u32x4{0u, 0u, 0u, 0u};
  wait_vmcnt<0>();  // the query and weights are in: only key tiles are in flight below

  const uint16_t* kb_base = k_idx + static_cast<size_t>(b) * S_max * DI + g * (DI / 2);

  // rows past the end of a partial tile re-read the chunk's last key
  auto load_tile = [&](bf16x8 (&dst)[NC], int t0) {
    const uint16_t* kp = kb_base + static_cast<size_t>(min(t0 + col, end - 1)) * DI;
#pragma unroll
    for (int c = 0; c < NC; ++c) dst[c] = load_bf16x8(kp + 8 * c);
  };
  // fused variant: bounds of the order keys of the competing positions this lane has scored
  // (both lane halves hold the same score), for the selection's digit window
  uint32_t run_mn = 0xffffffffu, run_mx = 0u;
  auto score_tile = [&](const bf16x8 (&src)[NC], int t0) {
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < NC; ++c) acc = mfma32(qa[c], src[c], acc);
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) part += wr[r] * fmaxf(acc[r], 0.0f);
    const float score = sum_xor32(part);
    if (g == 0) stage[t0 - start + col] = score;  // t0 - start + col < keys_per_wg
    if constexpr (FUSED) {
      const uint32_t k = sel::order_key(score);
      const bool ok = t0 + col >= comp_a && t0 + col <= comp_z;
      run_mn = ok ? min(run_mn, k) : run_mn;
      run_mx = ok ? max(run_mx, k) : run_mx;
    }
  };

  // tiles of this wavefront: t0 + i * WG_STRIDE for i < ntiles; two per iteration, so both
  // register buffers have fixed roles and the loop has no exit in the middle
  int t = start + wave * kTileKeys;
  const int ntiles = t < end ? (end - t + WG_STRIDE - 1) / WG_STRIDE : 0;
  bf16x8 ka[NC], kc[NC];
  load_tile(ka, t);
  int i = 0;
  for (; i + 3 <= ntiles; i += 2) {  // both prefetches of an iteration are tiles of this wavefront
    load_tile(kc, t + WG_STRIDE);
    __builtin_amdgcn_sched_barrier(0);  // keep the whole prefetch ahead of the matrix-core work
    score_tile(ka, t);
    load_tile(ka, t + 2 * WG_STRIDE);
    __builtin_amdgcn_sched_barrier(0);
    score_tile(kc, t + WG_STRIDE);
    t += 2 * WG_STRIDE;
  }
  // the last one or two tiles, with no load past the end: nothing is left in flight for the
  // selection that follows to wait for
  if (i + 2 <= ntiles) {
    load_tile(kc, t + WG_STRIDE);
    __builtin_amdgcn_sched_barrier(0);
    score_tile(ka, t);
    score_tile(kc, t + WG_STRIDE);
  } else if (i < ntiles) {
    score_tile(ka, t);
  }
  __syncthreads();
  if constexpr (!FUSED) {
    float* srow = P.scores + static_cast<size_t>(row) * S_max + start;
    for (int i = threadIdx.x; i < end - start; i += THREADS) srow[i] = stage[i];
  } else {
    __shared__ uint32_t sh[sel::chunk_scratch_words<THREADS, STAGE_ITEMS>()];
    const int a = comp_a, z = comp_z;  // competing positions here
    uint32_t key[STAGE_ITEMS];  // 0: the position does not compete
#pragma unroll
    for (int j = 0; j < STAGE_ITEMS; ++j) {
      // read unconditionally (the dynamic LDS holds at least STAGE_ITEMS * THREADS words), so
      // no read waits behind a branch
      const float v = stage[j * THREADS + static_cast<int>(threadIdx.x)];
      const int s = start + j * THREADS + static_cast<int>(threadIdx.x);
      key[j] = (s >= a && s <= z) ? sel::order_key(v) : 0u;
    }
    sel::chunk_candidates<THREADS, STAGE_ITEMS, true>(
        key, z - a + 1, P.R, sel::list_cap(P.R), start, hist, sh,
        P.cand + static_cast<size_t>(blockIdx.x) * P.list_stride, P.count + blockIdx.x,
        P.range + 2 * blockIdx.x, run_mn, run_mx);
  }
}

constexpr int kQbWaves = 8;        // wavefronts per workgroup (two per SIMD)
constexpr int kQbRowsPerWave = 2;  // query rows per wavefront (4 at one wavefront per SIMD,
                                   // 416 registers, is 13% slower: nothing hides the barriers)
constexpr int kQbMinRows = 16;     // row count from which the query-blocked scan is used
constexpr int kDropOffset = 1 << 30;      // beyond any row: such stores are dropped

struct QbParams {
  const uint16_t* q_idx;
  const float* w;
  const uint16_t* k_idx;
  const int32_t* seqlens;
  int Lq, Hi, S_max;
  int nqb;        // query blocks per sequence
  int nkc;        // key chunks per sequence
  int kc_keys;    // keys per chunk (multiple of 32)
  float* scores;
};

// RPW * WAVES query rows x one key chunk; Di = 128 (16 units of 16 bytes per key).  RPW rows per
// wavefront share every key fragment read from LDS (RPW matrix-core steps per read).
template <int WAVES, int RPW>
__global__ __launch_bounds__(64 * WAVES, 1) void index_scores_qb_kernel(QbParams P) {
  constexpr int DI = 128, NC = DI / 16, UK = DI / 8;
  constexpr int THREADS = 64 * WAVES, ROWS = RPW * WAVES;
  constexpr int LOADS = kTileKeys * UK / THREADS;  // 16-byte pieces per thread per tile
  static_assert(LOADS * THREADS == kTileKeys * UK, "whole tiles per load round");
  static_assert(RPW >= 2, "the epilogue of one row runs beside the next row's matrix-core steps");
  __shared__ __attribute__((aligned(16))) u32x4 kt[4][kTileKeys * UK];  // ring of four 8 KB tiles
  const int kc = blockIdx.x % P.nkc;
  const int rest = blockIdx.x / P.nkc;
  const int qb = rest % P.nqb;
  const int b = rest / P.nqb;
  const int Lq = P.Lq, Hi = P.Hi, S_max = P.S_max;
  const int sl = P.seqlens[b];
  const int i_last = min(qb * ROWS + ROWS - 1, Lq - 1);
  const int pmax = min(sl - Lq + i_last, S_max - 1);  // position of the block's last row
  const int start = kc * P.kc_keys;
  if (start > pmax) return;
  const int end = min(start + P.kc_keys, pmax + 1);  // keys [start, end)
  const int ntiles = (end - start + kTileKeys - 1) / kTileKeys;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, g = lane >> 5;

  // this wavefront's RPW query rows: fragments, weights, positions
  // Scores go out through buffer stores whose range is the row's keys [0, p]: lanes past p (and
  // every lane of a step past the end) store out of range, which the hardware drops.  The store
  // is therefore unconditional, so the compiler's wait counts stay exact (a store behind a branch
  // makes it wait for the prefetch issued after it).
  bf16x8 qa[RPW][NC];
  float wr[RPW][16];
  __amdgpu_buffer_rsrc_t rs[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const int i = qb * ROWS + RPW * wave + q;
    const bool ok = i < Lq;
    const size_t row = static_cast<size_t>(b) * Lq + min(i, Lq - 1);
    const int pq = ok ? min(sl - Lq + i, S_max - 1) : -1;  // keys s <= pq are scored
    rs[q] = __builtin_amdgcn_make_buffer_rsrc(P.scores + row * S_max, 0, 4 * (pq + 1), kBufferFlags);
    const uint16_t* qp = P.q_idx + (row * Hi + min(col, Hi - 1)) * DI + g * (DI / 2);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 v = load_bf16x8(qp + 8 * c);
      qa[q][c] = col < Hi ? v : zero_bf16x8();
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = acc_row(r, g);
      const float v = P.w[row * Hi + min(h, Hi - 1)];
      wr[q][r] = h < Hi ? v : 0.0f;
    }
  }

  // cooperative tile loads: piece j of thread t is unit t % 16 of key t / 16 + j * THREADS / 16;
  // in LDS, unit u of key k sits at slot u ^ (k % 16), so the fragment reads below hit 16
  // different bank groups
  const int lkey = tid >> 4, lunit = tid & 15;
  const uint16_t* kbase = P.k_idx + static_cast<size_t>(b) * S_max * DI + 8 * lunit;
  struct Piece { u32x4 v[LOADS]; };
  auto gload = [&](int t0) {
    Piece x;
#pragma unroll
    for (int j = 0; j < LOADS; ++j)
      x.v[j] = *reinterpret_cast<const u32x4*>(
          kbase + static_cast<size_t>(min(t0 + lkey + j * (THREADS / 16), S_max - 1)) * DI);
    return x;
  };
  auto lstore = [&](int slot, const Piece& x) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int k = lkey + j * (THREADS / 16);
      kt[slot][k * UK + (lunit ^ (k & (UK - 1)))] = x.v[j];
    }
  };
  auto barrier = [] {  // LDS only: the register prefetch stays in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // key fragments of the tile in LDS slot `slot`
  auto kread = [&](int slot, bf16x8 (&kb)[NC]) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
      kb[c] = __builtin_bit_cast(bf16x8, kt[slot][col * UK + ((g * NC + c) ^ (col & (UK - 1)))]);
  };
  // one epilogue element: weight x ReLU.  ReLU is a signed-integer max on the bit pattern:
  // negative floats (and -0) have negative patterns, so it gives max(x, 0) for finite x in one
  // instruction.
  auto relu_w = [&](int q, int r, float x) {
    return wr[q][r] * __int_as_float(max(__float_as_int(x), 0));
  };
  // head sum across the lane pair and the range-checked store of query row q on tile t (tiles
  // outside [0, ntiles) store nothing)
  // Tiles are stored in pairs: an even tile's sums wait in `held`, and with the odd tile after
  // it lanes g = 0 store the even tile's 32 keys and lanes g = 1 the odd tile's, one store of 64
  // consecutive keys.
  float held[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) held[q] = 0.0f;
  auto store_row = [&](int q, int t, float part, bool odd) {
    part = sum_xor32(part);
    if (!odd) {
      held[q] = part;
      return;
    }
    const int tt = t - 1 + g;
    const int key = start + tt * kTileKeys + col;  // < end within the last tile or dropped
    const int off = static_cast<unsigned>(tt) < static_cast<unsigned>(ntiles) ? 4 * key : kDropOffset;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(g ? part : held[q]), rs[q], off, 0, 0);
  };

  // Software pipeline.  Step t, with LDS slots rotating over 4:
  //   - reads tile t+1's fragments from LDS into registers (published at least one step earlier),
  //   - on even t, loads tiles t+4 and t+5 from memory into one of two register pairs,
  //   - runs row 0's 8 dependent matrix-core steps on tile t, each followed by two elements of
  //     the last row's epilogue of tile t-1; then row r's steps (r >= 1) next to row r-1's
  //     epilogue of tile t, one step behind, so that accumulator is complete,
  //   - on even t, writes tiles t+2 and t+3 (loaded two steps earlier) into their slots, then a
  //     barrier: the eight wavefronts meet every other step.  A slot is rewritten only after the
  //     barrier that follows its last read.
  // After a barrier the matrix cores start at once on fragments already in registers.  The
  // instruction order is fixed with scheduling barriers.  Four steps per iteration give every
  // register and slot a fixed role; steps past the end compute on clamped keys and store nothing.
  f32x16 acc[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) acc[q] = f32x16{};
  bf16x8 kx[NC], ky[NC];
  Piece ra[2], rb[2];
  ra[0] = gload(start);
  ra[1] = gload(start + kTileKeys);
  rb[0] = gload(start + 2 * kTileKeys);
  rb[1] = gload(start + 3 * kTileKeys);
  lstore(0, ra[0]);  // tile 0
  lstore(1, ra[1]);  // tile 1
  barrier();
  kread(0, kx);
  auto step = [&](int t, int slot, const bf16x8 (&kc)[NC], bf16x8 (&kn)[NC], Piece* st, Piece* ld,
                  bool t_odd) {
    kread(slot, kn);
    if (ld) {
      ld[0] = gload(start + (t + 4) * kTileKeys);
      ld[1] = gload(start + (t + 5) * kTileKeys);
    }
    {
      float p = 0.0f;  // last row, tile t-1
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc[0] = mfma32(qa[0][c], kc[c], c == 0 ? f32x16{} : acc[0]);
        p += relu_w(RPW - 1, 2 * c, acc[RPW - 1][2 * c]);
        p += relu_w(RPW - 1, 2 * c + 1, acc[RPW - 1][2 * c + 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      store_row(RPW - 1, t - 1, p, !t_odd);
    }
#pragma unroll
    for (int q = 1; q < RPW; ++q) {
      float p = 0.0f;  // row q - 1, tile t
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc[q] = mfma32(qa[q][c], kc[c], c == 0 ? f32x16{} : acc[q]);
        if (c > 0) {
          p += relu_w(q - 1, 2 * c - 2, acc[q - 1][2 * c - 2]);
          p += relu_w(q - 1, 2 * c - 1, acc[q - 1][2 * c - 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      p += relu_w(q - 1, 14, acc[q - 1][14]);
      p += relu_w(q - 1, 15, acc[q - 1][15]);
      store_row(q - 1, t, p, t_odd);
    }
    if (st) {
      lstore((slot + 1) & 3, st[0]);
      lstore((slot + 2) & 3, st[1]);
      barrier();
    }
  };
  // the last row stores tile t - 1 at step t, so its pair (ntiles - 1, ntiles) needs step
  // ntiles + 1
  for (int t = 0; t <= ntiles + 1; t += 4) {
    step(t, 1, kx, ky, rb, ra, false);
    step(t + 1, 2, ky, kx, nullptr, nullptr, true);
    step(t + 2, 3, kx, ky, ra, rb, false);
    step(t + 3, 0, ky, kx, nullptr, nullptr, true);
  }
}

template <int WAVES, int RPW>
hipError_t launch_qb(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                     const int32_t* seqlens, int B, int Lq, int Hi, int S_max, float* scores,
                     hipStream_t stream) {
  constexpr int ROWS = RPW * WAVES;
  QbParams Q{};
  Q.q_idx = q_idx;
  Q.w = w;
  Q.k_idx = k_idx;
  Q.seqlens = seqlens;
  Q.Lq = Lq;
  Q.Hi = Hi;
  Q.S_max = S_max;
  Q.nqb = (Lq + ROWS - 1) / ROWS;
  Q.nkc = 8;  // one key chunk per XCD
  Q.kc_keys = ((S_max + Q.nkc - 1) / Q.nkc + kTileKeys - 1) / kTileKeys * kTileKeys;
  Q.nkc = (S_max + Q.kc_keys - 1) / Q.kc_keys;
  Q.scores = scores;
  const long grid = static_cast<long>(B) * Q.nqb * Q.nkc;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((index_scores_qb_kernel<WAVES, RPW>), dim3(static_cast<unsigned>(grid)),
                     dim3(64 * WAVES), 0, stream, Q);
  return hipGetLastError();
}

// Keys per workgroup: about 512 workgroups (two per CU, all resident at once), whole workgroup
// steps per chunk (long chunks amortise the query/weight loads and the ramp of each workgroup),
// at most 8192 keys (the LDS score stage).  The fused call also keeps a row to at most 16
// candidate lists where the cap allows, so one merge takes them all (decode_32k: 16 chunks of 2048 keys, 14 us for its merge, against 64
// chunks of 512 keys and two merge levels, 23 us; decode_1m: 8192-key chunks scan 2% faster than
// 7680-key ones).
int keys_per_workgroup(long rows, int S_max, bool fused) {
  long per = (rows * S_max + 511) / 512;
  if (fused) per = std::max<long>(per, std::max<long>((S_max + 127) / 128, (S_max + 15) / 16));
  per = ((per + kWgStride - 1) / kWgStride) * kWgStride;
  if (per < kWgStride) per = kWgStride;
  if (per > kMaxKeysPerWg) per = kMaxKeysPerWg;
  return static_cast<int>(per);
}

template <int DI, bool FUSED, int THREADS>
hipError_t launch_kernel(const IndexParams& P, long grid, hipStream_t stream) {
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  size_t lds = static_cast<size_t>(P.keys_per_wg) * sizeof(float);
  if (FUSED) {
    lds += static_cast<size_t>(2 * sel::kBins) * sizeof(uint32_t);  // the selection's histogram
    const hipError_t err = hipFuncSetAttribute(
        reinterpret_cast<const void*>(index_scores_kernel<DI, FUSED, THREADS>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL((index_scores_kernel<DI, FUSED, THREADS>), dim3(static_cast<unsigned>(grid)),
                     dim3(THREADS), lds, stream, P);
  return hipGetLastError();
}

// wide: 512-thread workgroups (fused launches only; keys_per_wg a multiple of their step)
template <bool FUSED>
hipError_t launch_any(const IndexParams& P, int Di, long grid, hipStream_t stream, bool wide = false) {
  if (FUSED && wide) {
    switch (Di) {
      case 32: return launch_kernel<32, FUSED, kWideThreads>(P, grid, stream);
      case 64: return launch_kernel<64, FUSED, kWideThreads>(P, grid, stream);
      case 128: return launch_kernel<128, FUSED, kWideThreads>(P, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (Di) {
    case 32: return launch_kernel<32, FUSED, kThreads>(P, grid, stream);
    case 64: return launch_kernel<64, FUSED, kThreads>(P, grid, stream);
    case 128: return launch_kernel<128, FUSED, kThreads>(P, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

struct FusedPlan {
  int keys_per_wg = kWgStride, chunks = 1, stride = 1;  // stride: of the candidate lists
  long rows = 0, group = 1;
  size_t count_bytes = 0, range_bytes = 0, cand_bytes = 0, level1_bytes = 0;
};

FusedPlan fused_plan(int B, int Lq, int S_max, int topk, int init_tokens, int local_tokens) {
  FusedPlan pl;
  pl.rows = static_cast<long>(B) * Lq;
  pl.keys_per_wg = keys_per_workgroup(pl.rows, S_max, true);
  pl.chunks = (S_max + pl.keys_per_wg - 1) / pl.keys_per_wg;
  pl.stride = std::max(1, sel::list_capacity(topk - init_tokens - local_tokens, pl.keys_per_wg));
  const size_t per_row = static_cast<size_t>(pl.chunks) * pl.stride * sizeof(uint2);
  pl.group = std::max<long>(1, std::min<long>(pl.rows, static_cast<long>(kFusedBudget / per_row)));
  pl.count_bytes = (static_cast<size_t>(pl.group) * pl.chunks * 4 + 255) & ~static_cast<size_t>(255);
  pl.range_bytes = (static_cast<size_t>(pl.group) * pl.chunks * 8 + 255) & ~static_cast<size_t>(255);
  pl.cand_bytes = static_cast<size_t>(pl.group) * per_row;
  pl.level1_bytes = topk_merge_level1_bytes(pl.group, pl.chunks, topk, init_tokens, local_tokens);
  return pl;
}

}  // namespace

hipError_t launch_index_scores(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                               const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max,
                               float* scores, hipStream_t stream) {
  const long rows = static_cast<long>(B) * Lq;
  if (Di == 128 && Lq >= kQbMinRows)  // prefill: query-blocked scan
    return launch_qb<kQbWaves, kQbRowsPerWave>(q_idx, w, k_idx, seqlens, B, Lq, Hi, S_max, scores, stream);
  IndexParams P{};
  P.q_idx = q_idx;
  P.w = w;
  P.k_idx = k_idx;
  P.seqlens = seqlens;
  P.Lq = Lq;
  P.Hi = Hi;
  P.S_max = S_max;
  P.keys_per_wg = keys_per_workgroup(rows, S_max, false);
  P.chunks_per_row = (S_max + P.keys_per_wg - 1) / P.keys_per_wg;
  P.scores = scores;
  return launch_any<false>(P, Di, rows * P.chunks_per_row, stream);
}

size_t index_topk_workspace_bytes(int B, int Lq, int S_max, int topk, int init_tokens, int local_tokens) {
  const FusedPlan pl = fused_plan(B, Lq, S_max, topk, init_tokens, local_tokens);
  return pl.count_bytes + pl.range_bytes + pl.cand_bytes + pl.level1_bytes + kWorkspaceAlign;
}

hipError_t launch_index_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                             const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max,
                             int topk, int init_tokens, int local_tokens, int32_t* indices,
                             int32_t* n_sel, void* workspace, hipStream_t stream) {
  const FusedPlan pl = fused_plan(B, Lq, S_max, topk, init_tokens, local_tokens);
  if (pl.chunks > topk_merge_max_chunks()) return hipErrorInvalidConfiguration;
  IndexParams P{};
  P.q_idx = q_idx;
  P.w = w;
  P.k_idx = k_idx;
  P.seqlens = seqlens;
  P.Lq = Lq;
  P.Hi = Hi;
  P.S_max = S_max;
  P.keys_per_wg = pl.keys_per_wg;
  P.chunks_per_row = pl.chunks;
  P.list_stride = pl.stride;
  P.topk = topk;
  P.init = init_tokens;
  P.local = local_tokens;
  P.R = topk - init_tokens - local_tokens;
  char* ws = align_workspace(workspace);
  P.count = reinterpret_cast<uint32_t*>(ws);
  P.range = reinterpret_cast<uint32_t*>(ws + pl.count_bytes);
  P.cand = reinterpret_cast<uint2*>(ws + pl.count_bytes + pl.range_bytes);
  void* level1 = pl.level1_bytes ? ws + pl.count_bytes + pl.range_bytes + pl.cand_bytes : nullptr;
  for (long r0 = 0; r0 < pl.rows; r0 += pl.group) {
    const long g = std::min(pl.group, pl.rows - r0);
    P.row0 = static_cast<int>(r0);
    // a launch too small to fill the chip runs 8-wavefront workgroups (one per CU either way)
    const bool wide = g * pl.chunks <= kWideMaxGrid && pl.keys_per_wg % (kTileKeys * kWideThreads / 64) == 0;
    hipError_t err = launch_any<true>(P, Di, g * pl.chunks, stream, wide);
    if (err != hipSuccess) return err;
    err = launch_topk_merge(seqlens, Lq, S_max, topk, init_tokens, local_tokens, static_cast<int>(r0),
                            static_cast<int>(g), pl.chunks, pl.stride, P.count, P.range, P.cand,
                            level1, indices, n_sel, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace lsa
