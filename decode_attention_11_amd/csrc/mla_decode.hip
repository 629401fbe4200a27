// Paged absorbed-MLA decode for gfx950: plan, partial attention, split combine.
//
// What one call computes is stated in include/mla_decode.h (per-row causal
// bounds from the global lengths, round-robin rank-local keys, softmax over
// 576-wide scores, 512-wide values, LSE in base e or 2).
//
// Work decomposition.  The rows of request b are its q_len*H (query token,
// head) pairs, row = j*H + h, cut into row tiles.  Each (request, row tile)
// group must attend to n_b keys, n_b being the bound of its last query row.
// All groups' keys are laid end to end (units ordered by request, row tile,
// key) and cut into G equal ranges, one per workgroup, so every CU gets the
// same number of keys whatever the length mix (a balanced split-KV).  A
// range that crosses group boundaries is processed as several pieces.  Each
// piece writes an fp32 partial (unnormalised O^T, running max in log2 units,
// softmax denominator) to the workspace; a combine kernel merges the pieces
// of each group and writes bf16 out and the LSE.  The idea of splitting keys
// across workgroups with a workspace is the split-KV of the trtllm-gen path
// (PR #54012 page, implementation breakdown: the non-DCP call keeps its
// multi-CTA KV counter buffer); the balanced range split is this library's.
//
// Two kernel families compute the partials.  M16 (16 rows per tile) serves
// single-token decode with up to 16 heads, the HBM-bound case; R128 (128
// rows per tile) serves multi-token and many-head requests, where the score
// and value products dominate.  Both stream key tiles through an LDS ring,
// compute S^T = K Q^T so that each lane ends up holding keys of one query
// row, and feed P^T straight from registers into O^T += V^T P^T with V^T
// read from LDS by the transposing ds_read_b64_tr_b16.  The running max is a
// reference that only moves when a row's max grows by more than 2^8, so the
// accumulators are rarely rescaled (the exponentials stay <= 256, exact in
// fp32 and in bf16 range).  P enters P*V rounded to bf16; the output is
// normalised by the sum of those same rounded values (a row dominated by one
// key then reproduces that key's value row instead of being off by the
// rounding of its weight), while the LSE uses the fp32 sum.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "mla_decode.h"
#include "mla_device.h"

using namespace mla;

namespace {

struct DecodeArgs {
  const uint8_t* q;        // bf16 [B, Q, H, 576]
  const uint8_t* kv;       // bf16 [num_blocks, bs, 576]
  const int32_t* bt;       // [B, max_blocks]
  const int32_t* seq_lens; // [B]
  const int32_t* glob;     // [B] or null
  const int32_t* qsl;      // [B+1] token offsets of the requests (varlen), or null: Q tokens each
  int B, Q, H, R;          // Q: (largest) tokens per request, R = Q*H rows
  int num_blocks, bs, max_blocks;
  int bs_shift;            // log2(bs) when bs is a power of two, else -1
  int W, rank, causal;
  int I;                   // cp_interleave: positions go to ranks in segments of I
  float scale_log2;        // softmax scale (times the FP8 cache scale) times log2(e)
  float out_scale;         // output factor: the FP8 cache scale, 1 for bf16
  int kv_fp8;              // KV rows are 576 E4M3 bytes instead of 576 bf16
  int lse_base;
  int n_rt;                // row tiles per request (1 with per-tile ranges)
  int vrt;                 // per-tile ranges: row tiles per request, else 0
  int rows_tile;           // rows per row tile
  int ovh;                 // work units charged per piece on top of its keys
  int kalign;              // piece boundaries fall on multiples of this many keys (1 or 32)
  int nbund;               // balanced key ranges (bundles)
  int wa, wb;              // weights of the first and second half of the ranges
  int G;                   // partial workgroups: nbund * n_rt, one per (bundle, row tile)
  int64_t* prefix;         // [B+1] unit offsets of the requests ([B*vrt+1] of the (request, row tile) items)
  float* partials;         // [(nbund + B) * n_rt] slots
  uint16_t* out;           // bf16 [B*R, 512]
  float* lse;              // [B*R] or null
};

// Work units of a request: its keys plus a fixed overhead (the query rows'
// load and the partial's store), so that ranges crossing a request boundary
// get fewer keys.  Requests without keys cost nothing.  The units are those
// of one row tile: every row tile of a request has the same keys.
__device__ __forceinline__ int64_t request_units(const DecodeArgs& a, int nb) {
  return nb > 0 ? (int64_t)nb + a.ovh : 0;
}

// Partial slot of bundle j's piece of request bb, row tile rt.  For a fixed
// row tile, the bundles cover the requests in order, so j + bb never repeats.
// With per-tile ranges, range j's piece of item v = bb * vrt + rt: the ranges
// cover the items in order, so j + v never repeats either.
__device__ __forceinline__ int64_t piece_slot(const DecodeArgs& a, int j, int bb, int rt) {
  return a.vrt ? (int64_t)j + (int64_t)bb * a.vrt + rt : ((int64_t)j + bb) * a.n_rt + rt;
}

// Work items the ranges cut: the requests, or with per-tile ranges the
// (request, row tile) pairs, request by request.
__device__ __forceinline__ int work_items(const DecodeArgs& a) { return a.vrt ? a.B * a.vrt : a.B; }

// Query tokens of request b and the index of its first one: Q each, or
// from the token offsets of a varlen batch.
__device__ __forceinline__ void request_tokens(const DecodeArgs& a, int b, int& q_len, int& q_base) {
  if (a.qsl) {
    q_base = gload_i32(a.qsl + b);
    q_len = gload_i32(a.qsl + b + 1) - q_base;
  } else {
    q_base = b * a.Q;
    q_len = a.Q;
  }
}

// Key count of the largest row (the last query row sees the whole global
// length, whatever the query length), local length and global length of
// work item v (request v, or with per-tile ranges request v / vrt); zeros
// past the items, for a request without query tokens and for a row tile
// past its request's rows.
__device__ __forceinline__ void request_info(const DecodeArgs& a, int v, int& nb, int& seq, int& tot) {
  nb = seq = tot = 0;
  const int b = a.vrt ? v / a.vrt : v;
  if (v < work_items(a)) {
    seq = gload_i32(a.seq_lens + b);
    tot = a.glob ? gload_i32(a.glob + b) : seq;
    nb = row_bound(seq, tot, 1, 0, a.W, a.rank, a.I, a.causal);
    if (a.qsl) {
      const int ql = gload_i32(a.qsl + b + 1) - gload_i32(a.qsl + b);
      if (ql == 0 || (a.vrt && (v - b * a.vrt) * a.rows_tile >= ql * a.H)) nb = 0;
    }
  }
}

// Workgroups are dispatched to the 8 XCDs round-robin (blockIdx % 8).
// Numbered this way, consecutive indices sit on one XCD; with G/8 a multiple
// of n_rt, the n_rt workgroups of one bundle (the row tiles of the same keys,
// read at the same time) share that XCD's L2.
__device__ __forceinline__ int xcd_range_index(int block, int G) {
  return (G % 8 == 0) ? (block % 8) * (G / 8) + block / 8 : block;
}

// ---------------------------------------------------------------- in-kernel plan
// Every partial workgroup recomputes the request offsets itself (a block
// scan over seq_lens), so no separate planning launch is needed; workgroup 0
// also stores them for the combine kernel.
template <int NT>
__device__ __forceinline__ int64_t block_sum_i64(int64_t v, int64_t* s_red) {
  const int lane = lane_id_fresh(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int off = 32; off > 0; off >>= 1) v += shfl_i64(v, lane ^ off);
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  int64_t t = 0;
  for (int w = 0; w < NT / 64; ++w) t += s_red[w];
  return t;
}

template <int NT>
__device__ __forceinline__ int64_t block_incl_scan_i64(int64_t v, int64_t* s_red, int64_t& total) {
  const int lane = lane_id_fresh(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = shfl_i64(v, lane >= off ? lane - off : lane);
    if (lane >= off) v += y;
  }
  __syncthreads();
  if (lane == 63) s_red[wave] = v;
  __syncthreads();
  int64_t before = 0;
  total = 0;
  for (int w = 0; w < NT / 64; ++w) {
    const int64_t x = s_red[w];
    if (w < wave) before += x;
    total += x;
  }
  return before + v;
}

// ---------------------------------------------------------------- work ranges
template <int NT>
struct PlanLds {
  int64_t red[NT / 64];
  int64_t excl[NT];
  int nb[NT], seq[NT], tot[NT];
  int first_last[2][NT / 64];  // per wave: the first and last overlapping request (or sentinels)
};

// The key at which a range boundary x units past a request's overhead falls
// (0 .. nb): rounded down to a multiple of kalign, so that with 32 every
// 32-key tile of a piece lies in one block of a block size that 32 divides.
// Both pieces beside a boundary round it the same way.
__device__ __forceinline__ int piece_key(int64_t x, int nb, int kalign) {
  return x <= 0 ? 0 : x >= nb ? nb : (int)x & -kalign;
}

// The piece of request bb (unit offset pb, nbb keys) inside [u0, u1): the
// request's units are ovh overhead units, then one per key.
template <class F>
__device__ __forceinline__ void request_piece(const DecodeArgs& a, int bb, int64_t pb, int nbb, int sq, int tt,
                                              int64_t u0, int64_t u1, int rt, F&& piece) {
  if (nbb == 0) return;  // no keys: no units, no piece
  const int k0 = __builtin_amdgcn_readfirstlane(piece_key(u0 - pb - a.ovh, nbb, a.kalign));
  const int k1 = __builtin_amdgcn_readfirstlane(piece_key(u1 - pb - a.ovh, nbb, a.kalign));
  if (k1 <= k0) return;  // the range holds only the request's overhead units (or under kalign keys)
  if (a.vrt) {
    // item bb is row tile bb % vrt of request bb / vrt
    const int b = bb / a.vrt;
    piece(b, bb - b * a.vrt, k0, k1, sq, tt);
  } else {
    piece(bb, rt, k0, k1, sq, tt);
  }
}

// The requests' units are laid end to end and cut into nbund balanced
// ranges; bundle j's range is processed by n_rt workgroups, one per row tile.
// Calls piece(bb, rt, k0, k1, seq, tot) for every request that overlaps
// bundle j's range, in order, with the request's keys [k0, k1) inside the
// range.  Workgroup (0, 0) also stores the request offsets for the combine
// kernel.  All arguments of piece() are wave-uniform.  The workgroup scans
// the requests in chunks of NT, reading each length once per chunk (with up
// to NT requests one scan gives both the total and the offsets).
// A 64-bit value that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// What the plan keeps across the pieces is wave-uniform (scalar registers)
// or in LDS: a per-lane value live across the piece loop would be spilled,
// and each reload waits for every vector-memory operation in flight.
template <int NT, class F>
__device__ __forceinline__ void for_each_piece(const DecodeArgs& a, int j, int rt, PlanLds<NT>& pl, F&& piece) {
  const int tid = threadIdx.x;
  int64_t T, total0;
  {
    // chunk 0's offsets and lengths go to LDS for the first pass below
    int nb, seq, tot;
    request_info(a, tid, nb, seq, tot);
    int64_t t0;
    const int64_t incl0 = block_incl_scan_i64<NT>(request_units(a, nb), pl.red, t0);
    pl.excl[tid] = incl0 - request_units(a, nb);
    pl.nb[tid] = nb;
    pl.seq[tid] = seq;
    pl.tot[tid] = tot;
    total0 = uniform_i64(t0);
    T = total0;
    for (int base = NT; base < work_items(a); base += NT) {
      int nb2, seq2, tot2;
      request_info(a, base + tid, nb2, seq2, tot2);
      T += uniform_i64(block_sum_i64<NT>(request_units(a, nb2), pl.red));
    }
  }
  const int64_t u0 = uniform_i64(range_start(j, T, a.nbund, a.wa, a.wb));
  const int64_t u1 = uniform_i64(range_start(j + 1, T, a.nbund, a.wa, a.wb));

  int64_t carry = 0;
  for (int base = 0; base < work_items(a); base += NT) {
    int64_t chunk_total = total0;
    if (base > 0) {
      int nb, seq, tot;
      request_info(a, base + tid, nb, seq, tot);
      int64_t t;
      const int64_t incl = block_incl_scan_i64<NT>(request_units(a, nb), pl.red, t);
      chunk_total = uniform_i64(t);
      pl.excl[tid] = incl - request_units(a, nb) + carry;
      pl.nb[tid] = nb;
      pl.seq[tid] = seq;
      pl.tot[tid] = tot;
    }
    const int b = base + tid;
    const int64_t excl = pl.excl[tid];
    const int64_t x = request_units(a, pl.nb[tid]);
    const int64_t incl = excl + x;
    if (j == 0 && rt == 0 && b < work_items(a)) {
      a.prefix[b + 1] = incl;
      if (b == 0) a.prefix[0] = 0;
    }
    // the requests overlapping the range are contiguous: each wave finds its
    // first and last one by ballot, one barrier publishes them
    const uint64_t hit = __ballot(x > 0 && excl < u1 && incl > u0);
    const int wv = tid >> 6;
    if ((tid & 63) == 0) {
      pl.first_last[0][wv] = hit ? 64 * wv + __builtin_ctzll(hit) : 0x7fffffff;
      pl.first_last[1][wv] = hit ? 64 * wv + 63 - __builtin_clzll(hit) : -1;
    }
    __syncthreads();
    int first = 0x7fffffff, last = -1;
#pragma unroll
    for (int v = 0; v < NT / 64; ++v) {
      first = min(first, pl.first_last[0][v]);
      last = max(last, pl.first_last[1][v]);
    }
    first = __builtin_amdgcn_readfirstlane(first);
    last = __builtin_amdgcn_readfirstlane(last);
    carry += chunk_total;

    for (int i = first; i <= last; ++i)
      request_piece(a, __builtin_amdgcn_readfirstlane(base + i), uniform_i64(pl.excl[i]),
                    __builtin_amdgcn_readfirstlane(pl.nb[i]), __builtin_amdgcn_readfirstlane(pl.seq[i]),
                    __builtin_amdgcn_readfirstlane(pl.tot[i]), u0, u1, rt, piece);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- LDS ring loads
// Both kernel families stream key tiles into an LDS ring with direct
// global->LDS loads (global_load_lds_dwordx4) issued from inline assembly and
// waited on with explicit counts: the compiler does not know these loads, so
// it neither drains them at every barrier nor serialises LDS reads behind
// them.  Every loop iteration issues the same number of them (masked keys
// read a zero row), which keeps the counts static.

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  // 64 lanes x 16 bytes from per-lane global addresses to lds_base + 16*lane
  // one wait state between the scalar write of M0 and the LDS-DMA load that
  // reads it (the compiler's hazard checker does not look inside the asm)
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(base)
               : "memory", "m0");
}

// A zero latent row: keys outside the piece (or with an invalid block id)
// are loaded from here, so every lane issues the same loads and the V rows
// of masked keys are exact zeros (0 * NaN garbage would poison P*V).
__device__ __attribute__((aligned(64))) const uint4 kZeroRow[ROW_BYTES / 16] = {};

__device__ __forceinline__ int block_of(const DecodeArgs& a, int t) {
  return a.bs_shift >= 0 ? (t >> a.bs_shift) : t / a.bs;
}

// Row address of local key t (block-table entries of blocks e0.. in bt_lds),
// or the zero row when t >= k1 or the block id is invalid.
__device__ __forceinline__ const uint8_t* ring_row(const DecodeArgs& a, const int* bt_lds, int e0, int t, int k1) {
  const uint8_t* rowp = reinterpret_cast<const uint8_t*>(kZeroRow);
  asm volatile("" : "+v"(rowp));
  if (t < k1) {
    const int vb = block_of(a, t);
    const int blk = bt_lds[vb - e0];
    if ((unsigned)blk < (unsigned)a.num_blocks) rowp = a.kv + ((int64_t)blk * a.bs + (t - vb * a.bs)) * ROW_BYTES;
  }
  return rowp;
}

// Stage layout shared by both families: a stage holds 32 key rows of 1152
// bytes, unpadded, row r at byte 1152*r.  The 16-byte chunks of a row are
// swizzled: logical chunk c of row r sits at (c & ~7) | ((c ^ f(r)) & 7),
// f(r) = g((r >> 1) & 7) with g(v) = (v >> 1) | ((v & 1) << 2).  Rows are
// 1152 bytes (8 mod 16 in 16-byte bank groups), so odd rows already land on
// the other half of the banks; f is a permutation over even (and over odd)
// rows, which makes the score reads (8 consecutive rows, one chunk)
// conflict-free, and f(4u) ^ f(4u+2) = 4, which does the same for the
// transposed V reads (4 rows x 2-4 chunks).
__device__ __forceinline__ int ring_swz(int r) {
  const int v = (r >> 1) & 7;
  return (v >> 1) | ((v & 1) << 2);
}

constexpr int RING_TILE = 32;                          // key rows per stage
constexpr int RING_STAGE = RING_TILE * ROW_BYTES;      // 36 KiB
constexpr int RING_DMA_PER_WAVE = 9;                   // 1 KiB load instructions per wave per stage
static_assert(RING_STAGE == 4 * RING_DMA_PER_WAVE * 1024, "a stage is exactly the four waves' loads");

// Wave w loads rows 8w..8w+7 of a stage with 9 instructions: instruction m,
// lane l fills stage byte 1024*(9w+m) + 16*l, i.e. row 8w + (64m+l)/72,
// physical chunk (64m+l)%72.  sel_off[m] (per lane, fixed) holds the logical
// byte offset of that chunk in its row and, in bit 15, whether the row is
// the higher of the two rows instruction m touches.
__device__ __forceinline__ void ring_dma_offsets(int (&sel_off)[RING_DMA_PER_WAVE], int wave, int lane) {
#pragma unroll
  for (int m = 0; m < RING_DMA_PER_WAVE; ++m) {
    const int cidx = 64 * m + lane;
    const int row_rel = cidx / 72, pch = cidx - 72 * (cidx / 72);
    const int c = (pch & ~7) | ((pch ^ ring_swz(8 * wave + row_rel)) & 7);
    sel_off[m] = 16 * c | ((row_rel != (64 * m) / 72) ? (1 << 15) : 0);
  }
}

// The 8 row addresses of a wave's share of a tile (lane k < 8 of rowp holds
// the global address of row 8w + k; the other lanes' values are ignored),
// made wave-uniform, and the stage they go to.
struct RingRows {
  uint64_t rows[8];
  uint32_t stage_lds;
};

__device__ __forceinline__ RingRows ring_rows(const uint8_t* rowp, uint32_t stage_lds) {
  RingRows rr;
  const uint64_t row64 = reinterpret_cast<uint64_t>(rowp);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)row64, j);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(row64 >> 32), j);
    rr.rows[j] = ((uint64_t)hi << 32) | lo;
  }
  rr.stage_lds = stage_lds;
  return rr;
}

// Load instruction m (0..8) of a wave's share.  Issuing the nine one at a
// time between MFMAs keeps the address unit busy in the background instead
// of stalling every wave behind a burst of 36 loads.
__device__ __forceinline__ void ring_issue_one(const RingRows& rr, int m, int wave,
                                               const int (&sel_off)[RING_DMA_PER_WAVE]) {
  const int rlo = (64 * m) / 72;
  const int rhi = (64 * m + 63) / 72;
  const int so = sel_off[m];
  // lanes in the higher row add the (uniform) distance between the two row
  // addresses; arithmetic rather than a select keeps the compiler from
  // turning it into a compare chain over all eight rows
  const uint64_t dist = rr.rows[rhi] - rr.rows[rlo];
  const uint64_t msk = (uint64_t)0 - (uint64_t)((uint32_t)so >> 15);
  dma16(reinterpret_cast<const void*>(rr.rows[rlo] + (dist & msk) + (so & 0x7fff)),
        rr.stage_lds + 1024 * (RING_DMA_PER_WAVE * wave + m));
}

// All nine loads of a wave's share at once.
__device__ __forceinline__ void ring_issue_all(const RingRows& rr, int wave, const int (&sel_off)[RING_DMA_PER_WAVE]) {
#pragma unroll
  for (int m = 0; m < RING_DMA_PER_WAVE; ++m) ring_issue_one(rr, m, wave, sel_off);
}

// ---------------------------------------------------------------- M16 partial
// Memory-bound family: up to 16 rows per request (single-token decode with up
// to 16 heads and similar), any block size.  256 threads = 4 waves per
// workgroup, one workgroup per CU.  32-key tiles stream through a 4-stage LDS
// ring (three tiles, 108 KiB, in flight per CU while one is computed).
//
// Work split.  The 16 x 32 score tile S^T = K Q^T (v_mfma_f32_16x16x32_bf16,
// K from LDS, Q^T in registers) is cut four ways: wave w computes the keys of
// half w%2 over dims [288 (w/2), 288 (w/2) + 288), 9 MFMA steps.  The fp32
// partial tiles go through LDS and every wave adds them up in the same order,
// so all four waves hold bit-identical scores and the same online-softmax
// state; no merge is needed at the end.  The 512 value columns are split
// instead: wave w accumulates O^T[128w .. 128w+127][16 rows] (8 x 16 x 16
// fp32 tiles, 32 MFMA registers) with V^T from LDS by ds_read_b64_tr_b16.
//
// Stages use the shared swizzled row layout; the two 16-key halves are rows
// 0..15 and 16..31.  The dims are split between wave pairs by MFMA step
// parity (wave w takes k-steps 2k + w/2), which keeps every score read of a
// wave at one chunk position per row group.
//
// Pipeline.  The ring items are, per piece, the query rows (loaded through
// the ring like a key half, then read into registers) followed by the
// piece's key tiles, so neither a new request nor a new row tile drains the
// ring.  The block-table entries of all pieces of a batch are staged in LDS
// first; a batch ends when the LDS window or the segment list is full, and a
// piece too long for one window continues in the next batch with its state
// kept in registers.
constexpr int M16_THREADS = 256;
constexpr int M16_ROWS = 16;
constexpr int M16_TILE = RING_TILE;                // keys per tile
constexpr int M16_HALF = 16 * ROW_BYTES;           // bytes of a 16-key half of a stage
constexpr int M16_STAGE = RING_STAGE;              // 36 KiB
constexpr int M16_NS = 4;                          // ring stages
constexpr int M16_DMA_PER_WAVE = RING_DMA_PER_WAVE;
// FP8 cache: a ring item is 18 KiB (32 keys x 576 E4M3 bytes, or the 16
// bf16 query rows), 18 one-KiB loads: waves 0, 1 issue 5, waves 2, 3 issue 4
constexpr int M16F8_RAW = 18 * 1024;
constexpr int M16F8_NS = 3;
constexpr int M16F8_WG_PER_CU = 2;  // two workgroups per CU hide each other's latency chains
constexpr int M16F8_LOADS = M16F8_RAW / 1024;
constexpr int M16F8_ROW = D_QK;  // bytes of an E4M3 row
constexpr int M16_KSTEPS = 9;                      // 32-dim MFMA steps per wave (half of 576)
constexpr int M16_BT_WIN = 1024;                   // block-table entries held in LDS per batch
constexpr int M16_MAXSEG = 16;                     // segments per batch
constexpr int M16_DV_WAVE = D_V / 4;               // value columns per wave
constexpr float M16_RESCALE_LOG2 = 8.f;            // keep exponentials <= 2^8 between rescales
constexpr int M16_SEG_FIRST = 1;   // segment starts its (request, row tile) group: a Q item precedes it
constexpr int M16_SEG_LAST = 2;    // segment ends its group: the partial is written after its last tile


struct M16State {
  f32x4 o[8];
  float m_ref, l_part, l_out;  // l_part: sum of fp32 P (LSE); l_out: of bf16 P (output)
};

struct M16Seg {
  int bb, rt, ka, kb, seq, tot, e_base, flags;
  int q_len, q_base;  // the request's query tokens and its first token's index
};

// Ring position: segment s (with its descriptor), tile j (-1: the segment's
// Q item).  s >= nseg: past the end.
struct M16Cursor {
  int s, j, nt;
  M16Seg d;
};

__device__ __forceinline__ void m16_load_seg(M16Cursor& c, const M16Seg* segs, int nseg) {
  if (c.s >= nseg) return;
  const M16Seg d = segs[c.s];
  c.d.bb = __builtin_amdgcn_readfirstlane(d.bb);
  c.d.rt = __builtin_amdgcn_readfirstlane(d.rt);
  c.d.ka = __builtin_amdgcn_readfirstlane(d.ka);
  c.d.kb = __builtin_amdgcn_readfirstlane(d.kb);
  c.d.seq = __builtin_amdgcn_readfirstlane(d.seq);
  c.d.tot = __builtin_amdgcn_readfirstlane(d.tot);
  c.d.e_base = __builtin_amdgcn_readfirstlane(d.e_base);
  c.d.flags = __builtin_amdgcn_readfirstlane(d.flags);
  c.d.q_len = __builtin_amdgcn_readfirstlane(d.q_len);
  c.d.q_base = __builtin_amdgcn_readfirstlane(d.q_base);
  c.nt = (c.d.kb - c.d.ka + M16_TILE - 1) / M16_TILE;
  c.j = (c.d.flags & M16_SEG_FIRST) ? -1 : 0;
}

__device__ __forceinline__ void m16_advance(M16Cursor& c, const M16Seg* segs, int nseg) {
  if (c.s >= nseg) return;
  if (c.j + 1 < c.nt) {
    ++c.j;
  } else {
    ++c.s;
    m16_load_seg(c, segs, nseg);
  }
}

// Row addresses of this wave's share of ring item c (rows 8w..8w+7 of the
// stage; its 9 loads are issued from them).  A
// Q item loads the group's 16 query rows as rows 0..15 (waves 0 and 1);
// items past the end, and rows 16..31 of a Q item, load the zero row, so
// every wave issues 9 loads per item.
__device__ __forceinline__ RingRows m16_item_rows(const DecodeArgs& a, const int* bt_lds, int nseg,
                                                  const M16Cursor& c, uint32_t stage_lds, int wave, int lane) {
  const int r = 8 * wave + (lane & 7);  // the stage row this lane resolves (lanes 0..7 matter)
  const uint8_t* rowp = reinterpret_cast<const uint8_t*>(kZeroRow);
  asm volatile("" : "+v"(rowp));
  if (c.s < nseg) {
    if (c.j < 0) {
      const int qr = c.d.rt * M16_ROWS + r;
      if (r < M16_ROWS && qr < c.d.q_len * a.H) rowp = a.q + ((int64_t)c.d.q_base * a.H + qr) * ROW_BYTES;
    } else {
      const int t = c.d.ka + M16_TILE * c.j + r;
      if (t < c.d.kb) {
        const int vb = block_of(a, t);
        const int blk = bt_lds[c.d.e_base + vb];
        if ((unsigned)blk < (unsigned)a.num_blocks) rowp = a.kv + ((int64_t)blk * a.bs + (t - vb * a.bs)) * ROW_BYTES;
      }
    }
  }
  return ring_rows(rowp, stage_lds);
}

// ---- FP8 cache.  A key item holds 32 rows of 576 E4M3 bytes, row r at byte
// 576 r, unconverted; the computation widens its fragments to bf16 in
// registers (exactly: every E4M3 value is a bf16 value).  Rows are 144
// dwords apart (16 mod 32 banks), so the 16-byte chunks of each row are
// rotated: value chunk c < 32 of row r sits at (c + rot(r)) mod 32, rope
// chunk c >= 32 at 32 + (c + rot(r)) mod 4, with rot(r) = (r/2) mod 4 +
// 2 [r >= 16].  Then the 8 key rows of a transposed value read (keys 4g..4g+3
// and 16+4g..16+4g+3, one chunk) land on 8 different 16-byte bank groups,
// and the 16 key rows of a score read on every group twice.  The ring loads
// place the chunks: lane l of load g fills item chunk 64 g + l, and takes
// its bytes from whichever source chunk belongs there.
__device__ __forceinline__ int f8_rot(int r) { return ((r >> 1) & 3) + 2 * ((r >> 4) & 1); }
__device__ __forceinline__ int f8_pos(int r, int c) {
  return c < 32 ? (c + f8_rot(r)) & 31 : 32 + ((c + f8_rot(r)) & 3);
}
__device__ __forceinline__ int f8_chunk_at(int r, int q) {
  return q < 32 ? (q - f8_rot(r)) & 31 : 32 + ((q - f8_rot(r)) & 3);
}

// 8 E4M3 bytes to 8 bf16 values, byte e to element e
__device__ __forceinline__ bf16x8 f8x8_to_bf16(uint32_t x, uint32_t y) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(y, 1.0f, true);
  const bf16x4 lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4 hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Source addresses of this wave's loads of ring item c (load g = wave + 4m
// for m < 5 while g < 18), all resolved before the first is issued.  A Q
// item holds the group's 16 bf16 query rows in the swizzled layout of the
// bf16 ring; items past the end load zeros.
struct F8Loads {
  const uint8_t* p[5];
  uint32_t lds;
};

__device__ __forceinline__ F8Loads m16f8_loads(const DecodeArgs& a, const int* bt_lds, int nseg, const M16Cursor& c,
                                               uint32_t stage_lds, int wave, int lane) {
  F8Loads L;
  L.lds = stage_lds;
  const uint8_t* zero = reinterpret_cast<const uint8_t*>(kZeroRow);
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const int P = 64 * (wave + 4 * m) + lane;  // item chunk this lane fills
    const uint8_t* p = zero;
    asm volatile("" : "+v"(p));
    if (wave + 4 * m < M16F8_LOADS && c.s < nseg) {
      if (c.j < 0) {
        const int r = P / (ROW_BYTES / 16), q = P - (ROW_BYTES / 16) * r;
        const int ch = (q & ~7) | ((q ^ ring_swz(r)) & 7);
        const int qr = c.d.rt * M16_ROWS + r;
        p = (qr < c.d.q_len * a.H ? a.q + ((int64_t)c.d.q_base * a.H + qr) * ROW_BYTES : zero) + 16 * ch;
      } else {
        const int r = P / (M16F8_ROW / 16), q = P - (M16F8_ROW / 16) * r;
        const int ch = f8_chunk_at(r, q);
        const int t = c.d.ka + M16_TILE * c.j + r;
        p = zero + 16 * ch;
        if (t < c.d.kb) {
          const int vb = block_of(a, t);
          const int blk = bt_lds[c.d.e_base + vb];
          if ((unsigned)blk < (unsigned)a.num_blocks)
            p = a.kv + ((int64_t)blk * a.bs + (t - vb * a.bs)) * M16F8_ROW + 16 * ch;
        }
      }
    }
    L.p[m] = p;
  }
  return L;
}

__device__ __forceinline__ void m16f8_issue(const F8Loads& L, int m, int wave) {
  if (wave + 4 * m < M16F8_LOADS) dma16(L.p[m], L.lds + 1024 * (wave + 4 * m));
}

// One 32-key tile: this wave's quarter of S^T, the exchange of the partial
// tiles, online softmax with a lazily moved reference max, then this wave's
// quarter of O^T += V^T P^T.  qf holds the wave's 9 k-steps of Q^T.
template <bool F8, class Issue>
__device__ __forceinline__ void m16_compute(M16State& st, const bf16x8 (&qf)[M16_KSTEPS], const uint8_t* stage,
                                            uint8_t* xchg, float scale_log2, int ts, int k1, int nrow, int lane,
                                            int wave, Issue&& issue) {
  const int li = lane & 15, g = lane >> 4;
  // S^T[key][row] of half wave%2: lane (li, g) gets keys 4g+e for row li;
  // the K fragment of k-step kk = 2k + wave/2 is logical chunk 4kk + g of key
  // row li, i.e. physical byte 128k + 16*((4*(wave/2) + g) ^ f(row))
  const int kr = 16 * (wave & 1) + li;
  f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
  bf16x8 kf[M16_KSTEPS];
  // all nine reads first, then the MFMAs in two chains (one chain of nine
  // dependent MFMAs would wait out the MFMA latency at every step)
  if constexpr (F8) {
    // dims 64kk + 32(wave/2) + 8g .. +7 are E4M3 bytes 8(g%2) .. +7 of
    // chunk 4kk + 2(wave/2) + g/2
    const uint8_t* kp = stage + M16F8_ROW * kr + 8 * (g & 1);
    const int c0 = 2 * (wave >> 1) + (g >> 1);
    uint2 raw[M16_KSTEPS];
#pragma unroll
    for (int kk = 0; kk < M16_KSTEPS; ++kk)
      raw[kk] = *reinterpret_cast<const uint2*>(kp + 16 * f8_pos(kr, 4 * kk + c0));
#pragma unroll
    for (int kk = 0; kk < M16_KSTEPS; ++kk) kf[kk] = f8x8_to_bf16(raw[kk].x, raw[kk].y);
  } else {
    const uint8_t* kp = stage + ROW_BYTES * kr + 16 * ((4 * (wave >> 1) + g) ^ ring_swz(kr));
#pragma unroll
    for (int kk = 0; kk < M16_KSTEPS; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(kp + 128 * kk);
  }
  // one ring load of a later item per MFMA step (a burst of 36 after the
  // barrier would stall the waves behind the address unit)
#pragma unroll
  for (int kk = 0; kk < M16_KSTEPS; ++kk) {
    issue(kk);
    if (kk & 1)
      sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[kk], sb, 0, 0, 0);
    else
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[kk], sa, 0, 0, 0);
  }
  // exchange: xchg[w] holds wave w's partial tile in the accumulator layout
  *reinterpret_cast<f32x4*>(xchg + 1024 * wave + 16 * lane) = sa + sb;
  __syncthreads();
  const f32x4 p0 = *reinterpret_cast<const f32x4*>(xchg + 16 * lane);
  const f32x4 p1 = *reinterpret_cast<const f32x4*>(xchg + 1024 + 16 * lane);
  const f32x4 p2 = *reinterpret_cast<const f32x4*>(xchg + 2048 + 16 * lane);
  const f32x4 p3 = *reinterpret_cast<const f32x4*>(xchg + 3072 + 16 * lane);
  const f32x4 s0 = p0 + p2, s1 = p1 + p3;  // same order in every wave: identical scores
  float p[8];
  float mx = NEG_INF;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int t0 = ts + 4 * g + e, t1 = t0 + 16;
    p[e] = (t0 < k1 && t0 < nrow) ? s0[e] * scale_log2 : NEG_INF;
    p[4 + e] = (t1 < k1 && t1 < nrow) ? s1[e] * scale_log2 : NEG_INF;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) mx = fmaxf(mx, p[e]);
  // move the reference only when some row's max grew by more than 2^8 over it
  if (__ballot(mx > st.m_ref + M16_RESCALE_LOG2) != 0) {
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (mx > st.m_ref + M16_RESCALE_LOG2) {
      const float alpha = fast_exp2(st.m_ref - mx);
      st.l_part *= alpha;
      st.l_out *= alpha;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // in place on the accumulator register (a plain multiply makes the
          // register allocator copy every accumulator out of the MFMA
          // registers at each tile)
          float tmp;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(st.o[mt][i]), "=&v"(tmp) : "v"(alpha));
        }
      st.m_ref = mx;
    }
  }
  // masked scores are -inf and exp2(-inf) = 0; a row with no visible key
  // yet has only -inf scores and a -inf reference, so it subtracts 0
  const float m_sub = st.m_ref == NEG_INF ? 0.f : st.m_ref;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = fast_exp2(p[e] - m_sub);
    st.l_part += p[e];
  }
  // P^T as the B operand: contraction slot 8g+e is key 4g+e of half e/4
  const bf16x4 plo = to_bf16x4(p[0], p[1], p[2], p[3]);
  const bf16x4 phi = to_bf16x4(p[4], p[5], p[6], p[7]);
  const bf16x8 pf = __builtin_shufflevector(plo, phi, 0, 1, 2, 3, 4, 5, 6, 7);
  st.l_out = sum_bf16x8(pf, st.l_out);
  // V^T fragments: lane (li, g) of a transposed read points at key row
  // 16h + 4g + li/4, value columns 16T + 4(li%4) .. +3 (logical chunk
  // 2T + (li/2)%2, byte 8(li%2)) and receives column 16T + li of the 4 rows;
  // T = 8*wave + mt, so the chunk is 8(2*wave + mt/4) + 2(mt%4) + (li/2)%2
  if constexpr (F8) {
    // an 8-bit transposed read: in each 16-lane group, lanes 2e and 2e+1
    // address the two halves of block row e (key 4g+e, or 16+4g+e-4 for
    // e >= 4, as in P^T) of value chunk T = 8 wave + mt, and lane li receives
    // byte column li of the 8 rows
    const int e = li >> 1;
    const int key = e < 4 ? 4 * g + e : 12 + 4 * g + e;
    const uint8_t* vrow = stage + M16F8_ROW * key + 8 * (li & 1);
    const int vrot = f8_rot(key) + 8 * wave;
    i32x2 v[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      v[mt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vrow + 16 * ((vrot + mt) & 31)));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      st.o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f8x8_to_bf16((uint32_t)v[mt].x, (uint32_t)v[mt].y), pf,
                                                         st.o[mt], 0, 0, 0);
  } else {
    const int vr = 4 * g + (li >> 2);
    const int vsw = ring_swz(vr);  // equal for rows vr and 16 + vr
    const uint8_t* vrow = stage + ROW_BYTES * vr + 256 * wave + 8 * (li & 1);
    const uint8_t* vp[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) vp[q] = vrow + 16 * ((2 * q + ((li >> 1) & 1)) ^ vsw);
    i16x4 v[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      v[mt][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp[mt & 3] + 128 * (mt >> 2)));
      v[mt][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp[mt & 3] + M16_HALF + 128 * (mt >> 2)));
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const bf16x4 a0 = __builtin_bit_cast(bf16x4, v[mt][0]);
      const bf16x4 a1 = __builtin_bit_cast(bf16x4, v[mt][1]);
      st.o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7),
                                                         pf, st.o[mt], 0, 0, 0);
    }
  }
}

template <bool F8>
__global__ __launch_bounds__(M16_THREADS, F8 ? M16F8_WG_PER_CU : 1) void attn_m16_kernel(DecodeArgs a) {
  // bf16 cache: 4 stages of 36 KiB, one workgroup per CU.  FP8 cache: 3 of
  // 18 KiB (about 68 KiB of LDS in all, 236 VGPRs), two workgroups per CU,
  // each running its tile computation while the other waits on its loads.
  constexpr int NS = F8 ? M16F8_NS : M16_NS;
  constexpr int RAW = F8 ? M16F8_RAW : M16_STAGE;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * RAW];
  __shared__ __attribute__((aligned(16))) uint8_t xchg[4 * 1024];
  __shared__ int bt_lds[M16_BT_WIN];
  __shared__ M16Seg segs[M16_MAXSEG];
  __shared__ PlanLds<M16_THREADS> plan;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, g = lane >> 4;
  // With one row tile per request each key is read by one workgroup only:
  // ranges go in launch order (grouping them by XCD would concentrate slow
  // requests on a few XCDs).  With several row tiles, a bundle's workgroups
  // read the same keys and sit on one XCD, whose L2 then serves all but the
  // first read.
  const int wi = a.n_rt > 1 ? xcd_range_index(blockIdx.x, a.G) : (int)blockIdx.x;
  const int bund = wi / a.n_rt, tile = wi - bund * a.n_rt;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
  int sel_off[RING_DMA_PER_WAVE];  // per-lane constants of this wave's ring loads
  if constexpr (!F8) ring_dma_offsets(sel_off, wave, lane);
  auto f8_issue_all = [&](const F8Loads& L) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 5; ++m) m16f8_issue(L, m, wave);
  };

  // state of the group being computed; it survives batch boundaries
  bf16x8 qf[M16_KSTEPS];
#pragma unroll
  for (int kk = 0; kk < M16_KSTEPS; ++kk) qf[kk] = zero_bf16x8();
  M16State st;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) st.o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_ref = NEG_INF;
  st.l_part = 0.f;
  st.l_out = 0.f;
  int nrow = 0;
  int nseg = 0, nent = 0;  // segments and window entries of the batch being built

  auto run_batch = [&]() __attribute__((always_inline)) {
    if (nseg == 0) return;
    __syncthreads();  // window and segment list written
    M16Cursor ci{0, 0, 0, {}};
    m16_load_seg(ci, segs, nseg);
    int n_items = 0;
    for (int s = 0; s < nseg; ++s) {
      const int fl = __builtin_amdgcn_readfirstlane(segs[s].flags);
      const int ka = __builtin_amdgcn_readfirstlane(segs[s].ka), kb = __builtin_amdgcn_readfirstlane(segs[s].kb);
      n_items += ((fl & M16_SEG_FIRST) ? 1 : 0) + (kb - ka + M16_TILE - 1) / M16_TILE;
    }
    M16Cursor cc = ci;
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) {
      if constexpr (F8)
        f8_issue_all(m16f8_loads(a, bt_lds, nseg, ci, ring_lds + p * RAW, wave, lane));
      else
        ring_issue_all(m16_item_rows(a, bt_lds, nseg, ci, ring_lds + p * RAW, wave, lane), wave, sel_off);
      m16_advance(ci, segs, nseg);
    }
    for (int it = 0; it < n_items; ++it) {
      // item it landed (items it+1 .. it+NS-2 may still be in flight), and
      // after the barrier every wave is done with item it-1 ...
      if constexpr (F8) {
        if (wave < 2)
          WAIT_VMCNT(5 * (NS - 2));
        else
          WAIT_VMCNT(4 * (NS - 2));
      } else {
        WAIT_VMCNT(M16_DMA_PER_WAVE * (NS - 2));
      }
      __syncthreads();
      // ... so its stage can take item it+NS-1
      const uint32_t nxt_lds = ring_lds + ((it + NS - 1) % NS) * RAW;
      RingRows nxt;
      F8Loads nxt8;
      if constexpr (F8)
        nxt8 = m16f8_loads(a, bt_lds, nseg, ci, nxt_lds, wave, lane);
      else
        nxt = m16_item_rows(a, bt_lds, nseg, ci, nxt_lds, wave, lane);
      m16_advance(ci, segs, nseg);
      const uint8_t* stage = ring + (it % NS) * RAW;
      if (cc.j < 0) {
        // Q item: this wave's k-steps of Q^T (lane (li, g): dims
        // 32kk + 8g .. +7 of row li, kk = 2k + wave/2; stored like bf16 key
        // rows 0..15) into registers, and a fresh state
        const uint8_t* qp = stage + ROW_BYTES * li + 16 * ((4 * (wave >> 1) + g) ^ ring_swz(li));
#pragma unroll
        for (int kk = 0; kk < M16_KSTEPS; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 128 * kk);
        if constexpr (F8)
          f8_issue_all(nxt8);
        else
          ring_issue_all(nxt, wave, sel_off);
        const int my_row = cc.d.rt * M16_ROWS + li;
        nrow = my_row < cc.d.q_len * a.H
                   ? row_bound(cc.d.seq, cc.d.tot, cc.d.q_len, my_row / a.H, a.W, a.rank, a.I, a.causal)
                   : 0;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) st.o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m_ref = NEG_INF;
        st.l_part = 0.f;
        st.l_out = 0.f;
      } else {
        if constexpr (F8)
          m16_compute<true>(st, qf, stage, xchg, a.scale_log2, cc.d.ka + M16_TILE * cc.j, cc.d.kb, nrow, lane, wave,
                            [&](int kk) __attribute__((always_inline)) {
                              if (kk < 5) m16f8_issue(nxt8, kk, wave);
                            });
        else
          m16_compute<false>(st, qf, stage, xchg, a.scale_log2, cc.d.ka + M16_TILE * cc.j, cc.d.kb, nrow, lane,
                             wave, [&](int kk) __attribute__((always_inline)) { ring_issue_one(nxt, kk, wave, sel_off); });
        if (cc.j == cc.nt - 1 && (cc.d.flags & M16_SEG_LAST)) {
          // partial slot: wave w's O^T tiles T = 8w + mt in the accumulator
          // layout [T][lane][4] (one 16-byte store per lane and tile), then
          // per row m, the fp32 and the bf16 sums of P
          float l_row = st.l_part, lo_row = st.l_out;
          l_row += __shfl_xor(l_row, 16, 64);
          l_row += __shfl_xor(l_row, 32, 64);
          lo_row += __shfl_xor(lo_row, 16, 64);
          lo_row += __shfl_xor(lo_row, 32, 64);
          float* ps = a.partials + piece_slot(a, bund, cc.d.bb, cc.d.rt) * (M16_ROWS * D_V + 3 * M16_ROWS);
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
            *reinterpret_cast<f32x4*>(ps + ((M16_DV_WAVE / 16) * wave + mt) * 256 + 4 * lane) = st.o[mt];
          if (wave == 0 && g == 0) {
            ps[M16_ROWS * D_V + li] = st.m_ref;
            ps[M16_ROWS * D_V + M16_ROWS + li] = l_row;
            ps[M16_ROWS * D_V + 2 * M16_ROWS + li] = lo_row;
          }
        }
      }
      m16_advance(cc, segs, nseg);
    }
    WAIT_VMCNT(0);
    __syncthreads();  // the ring, the window and the segment list are free again
    nseg = 0;
    nent = 0;
  };

  for_each_piece<M16_THREADS>(a, bund, tile, plan, [&](int bb, int rt, int k0, int k1, int seq, int tot) {
    // append the piece (rows [16 rt, 16 rt + 16) of request bb, keys [k0, k1))
    // to the batch as one or more segments; a row tile past the request's
    // rows (a shorter query in a varlen batch) has nothing to compute
    int q_len, q_base;
    request_tokens(a, bb, q_len, q_base);
    q_len = __builtin_amdgcn_readfirstlane(q_len);
    q_base = __builtin_amdgcn_readfirstlane(q_base);
    if (rt * M16_ROWS >= q_len * a.H) return;
    const int32_t* btr = a.bt + (int64_t)bb * a.max_blocks;
    int flags = M16_SEG_FIRST;
    for (int ka = k0; ka < k1;) {
      if (nseg == M16_MAXSEG || M16_BT_WIN - nent < 2) run_batch();
      const int room = M16_BT_WIN - nent;
      const int64_t max_keys = (int64_t)(room - 1) * a.bs;  // any such key range spans <= room blocks
      const int kb = (int64_t)(k1 - ka) <= max_keys ? k1 : ka + (int)max_keys;
      const int e0 = block_of(a, ka), e1 = block_of(a, kb - 1);
      for (int e = e0 + tid; e <= e1; e += M16_THREADS)
        bt_lds[nent + e - e0] = e < a.max_blocks ? gload_i32(btr + e) : -1;
      if (tid == 0)
        segs[nseg] = M16Seg{bb, rt, ka, kb, seq, tot, nent - e0, flags | (kb == k1 ? M16_SEG_LAST : 0), q_len, q_base};
      ++nseg;
      nent += e1 - e0 + 1;
      ka = kb;
      flags = 0;
    }
  });
  run_batch();
}

// ---------------------------------------------------------------- R128 partial
// Compute-bound family: more than 16 rows per request (multi-token or many
// heads: 4 x 128 or 16 x 128 rows), any block size.  A workgroup
// owns 128 rows of one request and a key range; the 32-key tiles of the latent
// KV are shared by the four waves through a 3-stage LDS ring.
//
// Work split.  Scores and softmax: wave w owns rows 32w .. 32w+31 and
// computes S^T = K Q^T for them on v_mfma_f32_32x32x16_bf16 (K from LDS, Q^T
// in registers and LDS); each lane then holds 16 keys of one row.  The wave
// writes its bf16 P tile and a per-row rescale factor to LDS.  After one
// barrier, values are split by column instead: wave w accumulates
// O^T[128w .. 128w+127][all 128 rows] (16 32x32 fp32 blocks in the 256 MFMA
// accumulator registers) from V^T (ds_read_b64_tr_b16, its own 128 columns
// only) and P^T read back from LDS.  Every wave therefore reads each V
// column once per tile instead of all 512, and P crosses LDS once.
constexpr int R128_THREADS = 256;
constexpr int R128_ROWS = 128;
constexpr int R128_TILE = RING_TILE;          // keys per tile
constexpr int R128_ROWB = ROW_BYTES;          // LDS bytes per key row (unpadded; chunks are swizzled instead)
constexpr int R128_DMA_PER_WAVE = RING_DMA_PER_WAVE;
constexpr int R128_STAGE = RING_STAGE;        // 36 KiB
constexpr int R128_NS = 3;                    // ring stages
// The same kernel also runs tiles of 32 or 64 rows (requests of 17 to 64
// rows: fewer heads, a few query tokens), with NRB = rows / 32 row blocks:
// the score MFMAs of a row block are split by dims over the 4/NRB waves that
// share it, waves 0 .. NRB-1 add the slices and run the softmax, and every
// wave accumulates its 128 value columns for the NRB row blocks.
// Partial slot of a tile of `rows` rows: fp16 O, then m, l, lo per row and
// a power-of-two factor per (value-column quarter, row), fp32.
constexpr int r128_o_bytes(int rows) { return rows * D_V * 2; }
constexpr int r128_slot_bytes(int rows) { return r128_o_bytes(rows) + 7 * rows * 4; }
constexpr int R128_BT_WIN = 1024;             // block-table entries held in LDS per sub-piece
// Q^T k-steps (of 16 dims) kept in registers; the rest in LDS.
constexpr int R128_QREG = 28;
constexpr int R128_QLDS = 36 - R128_QREG;
constexpr int R128_PROW = 80;                 // LDS bytes per row of the P tile (64 + 16: conflict-free reads)
constexpr float R128_RESCALE_LOG2 = 8.f;


// Row addresses of this wave's share (rows 8w..8w+7) of tile [ts, ts+32).
__device__ __forceinline__ RingRows r128_tile_rows(const DecodeArgs& a, const int* bt_lds, int e0, int ts, int k1,
                                                   uint32_t stage_lds, int wave, int lane) {
  // lanes 0..7 resolve the row address of key ts + 8*wave + lane (or the zero row)
  const int k = lane & 7;
  const int t = ts + 8 * wave + k;
  const uint8_t* rowp = reinterpret_cast<const uint8_t*>(kZeroRow);
  asm volatile("" : "+v"(rowp));
  if (t < k1) {
    const int vb = block_of(a, t);
    const int blk = bt_lds[vb - e0];
    if ((unsigned)blk < (unsigned)a.num_blocks)
      rowp = a.kv + ((int64_t)blk * a.bs + (t - vb * a.bs)) * ROW_BYTES;
  }
  return ring_rows(rowp, stage_lds);
}

// An E4M3 tile of zeros: the source of every key past the piece or in an
// invalid block.
__device__ __attribute__((aligned(64))) const uint4 kZeroTileF8[M16F8_RAW / 16] = {};

// FP8 cache: what the loads of tile [ts, ts+32) need, all wave-uniform.
// The stage holds the tile's 32 E4M3 rows row-major (576 bytes each; the
// tile is widened before any fragment is read), filled by 18 one-KiB loads:
// load g (g = wave + 4m, m < 5, g < 18) copies stage bytes 1024 g .. +1023.
// With blocks of 32 keys or more the tile lies in at most two blocks, each
// holding its rows contiguously, so stage byte 16 P comes from base + 16 P
// with base = a (rows before `split`), b (rows from `split` on) or the zero
// tile (rows at or past `rows`): two compares per load instead of a
// block-table lookup per lane.  Smaller blocks look each row up at issue.
struct F8Tile {
  const uint8_t* a;
  const uint8_t* b;
  int split16, rows16;  // 576 * split and 576 * rows: byte bounds within the tile
  int ts, k1;
  uint32_t lds;
  bool rowwise;         // blocks under 32 keys
};

__device__ __forceinline__ F8Tile r128f8_tile(const DecodeArgs& a, const int* bt_lds, int e0, int ts, int k1,
                                              uint32_t stage_lds) {
  F8Tile T;
  const uint8_t* zero = reinterpret_cast<const uint8_t*>(kZeroTileF8);
  T.lds = stage_lds;
  T.ts = ts;
  T.k1 = k1;
  T.rowwise = a.bs < R128_TILE;
  const int rows = k1 - ts < 0 ? 0 : (k1 - ts > R128_TILE ? R128_TILE : k1 - ts);
  T.rows16 = M16F8_ROW * rows;
  T.a = T.b = zero;
  T.split16 = T.rows16;
  if (!T.rowwise && rows > 0) {
    const int vb = block_of(a, ts);
    const int off = ts - vb * a.bs;
    const int split = a.bs - off;  // rows of the tile in block vb
    T.split16 = M16F8_ROW * (split < rows ? split : rows);
    const int blk = __builtin_amdgcn_readfirstlane(bt_lds[vb - e0]);
    if ((unsigned)blk < (unsigned)a.num_blocks) T.a = a.kv + ((int64_t)blk * a.bs + off) * M16F8_ROW;
    if (split < rows) {
      const int blk2 = __builtin_amdgcn_readfirstlane(bt_lds[vb + 1 - e0]);
      // row r >= split of the tile is row r - split of block vb + 1
      if ((unsigned)blk2 < (unsigned)a.num_blocks) T.b = a.kv + ((int64_t)blk2 * a.bs - split) * M16F8_ROW;
    }
  }
  return T;
}

// Load m of this wave for tile T (nothing for g = wave + 4m >= 18): the
// two-block path, and the row-by-row one for blocks under 32 keys.
__device__ __forceinline__ void r128f8_issue(const F8Tile& T, int m, int wave, int lane) {
  const int g = wave + 4 * m;
  if (g >= M16F8_LOADS) return;
  const int b16 = 16 * (64 * g + lane);
  const uint8_t* src = (b16 < T.split16 ? T.a : T.b) + b16;
  if (b16 >= T.rows16) src = reinterpret_cast<const uint8_t*>(kZeroTileF8) + b16;
  dma16(src, T.lds + 1024 * g);
}

__device__ __forceinline__ void r128f8_issue_rowwise(const DecodeArgs& a, const int* bt_lds, int e0, const F8Tile& T,
                                                     int m, int wave) {
  const int g = wave + 4 * m;
  if (g >= M16F8_LOADS) return;
  // the lane index afresh: the per-lane row and chunk split would otherwise
  // be hoisted out of the tile loop and spilled
  const int P = 64 * g + lane_id_fresh();
  const int r = P / (M16F8_ROW / 16), ch = P - (M16F8_ROW / 16) * r;
  const int t = T.ts + r;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(kZeroTileF8) + 16 * P;
  if (t < T.k1) {
    const int vb = block_of(a, t);
    const int blk = bt_lds[vb - e0];
    if ((unsigned)blk < (unsigned)a.num_blocks)
      src = a.kv + ((int64_t)blk * a.bs + (t - vb * a.bs)) * M16F8_ROW + 16 * ch;
  }
  dma16(src, T.lds + 1024 * g);
}

// A landed E4M3 tile (32 rows of 576 bytes, row-major) widened into a bf16
// tile in the ring's swizzled layout, once per workgroup: lane l of wave w
// converts row 8w + l/8, bytes 72 (l%8) .. +71, nine 8-byte groups (item i:
// bytes 72 (l%8) + 8i) that each become one 16-byte bf16 chunk (logical
// chunk c at physical chunk (c & ~7) | ((c ^ f(r)) & 7)).  E4M3 values are
// exact in bf16, and zero rows stay zero.  The read and the write of an item
// are separate steps so that they can be spread over other work.
__device__ __forceinline__ uint2 r128f8_widen_read(const uint8_t* src, int wave, int lane, int i) {
  const int r = 8 * wave + (lane >> 3), c = 9 * (lane & 7) + i;
  return *reinterpret_cast<const uint2*>(src + r * M16F8_ROW + 8 * c);
}
__device__ __forceinline__ void r128f8_widen_write(uint8_t* dst, int wave, int lane, int i, uint2 x) {
  const int r = 8 * wave + (lane >> 3), c = 9 * (lane & 7) + i;
  const int fr = ring_swz(r);
  *reinterpret_cast<bf16x8*>(dst + r * R128_ROWB + 16 * ((c & ~7) | ((c ^ fr) & 7))) = f8x8_to_bf16(x.x, x.y);
}
__device__ __forceinline__ void r128f8_widen(const uint8_t* src, uint8_t* dst, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 9; ++i) r128f8_widen_write(dst, wave, lane, i, r128f8_widen_read(src, wave, lane, i));
}

// Per-lane LDS byte offsets inside a stage, fixed for the whole kernel (the
// stage base is one wave-uniform value per tile, so every address costs a
// single add).
struct R128LaneOff {
  uint32_t k[4];      // K fragment of the wave's k-step kb0 + 4a + b: k[b] + 128a
  uint32_t v[2][2];   // V^T transposed reads [rd][d%2]: + 16*1152*ks + 128*(d/2)
};

// kb0: the wave's first k-step (0, or the first of its slice of the 576
// dims when the scores of a row block are split across waves)
__device__ __forceinline__ R128LaneOff r128_lane_offsets(int lane, int wave, int kb0 = 0) {
  R128LaneOff lo;
  const int r = lane & 31, h = lane >> 5;
  // k-step kk reads logical chunk c = 2kk + h of row r, at physical chunk
  // (c & ~7) | ((c ^ f(r)) & 7); four k-steps further is 8 chunks (128 bytes)
  // further in both
  const int fk = ring_swz(r);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int c = 2 * (kb0 + b) + h;
    lo.k[b] = r * R128_ROWB + 16 * ((c & ~7) | ((c ^ fk) & 7));
  }
  // V^T: lane (q, i16) of a transposed read covers key row 8h + 4rd + i16/4
  // (+16ks), logical chunk 4D + 2(q%2) + (i16%4)/2 for D = 4w + d, byte
  // 8(i16%2)
  const int q = lane >> 4, i16 = lane & 15;
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int vr = 8 * h + 4 * rd + (i16 >> 2);
    const int fs = ring_swz(vr);
#pragma unroll
    for (int dp = 0; dp < 2; ++dp)
      lo.v[rd][dp] = vr * R128_ROWB + 256 * wave + 8 * (i16 & 1) +
                     16 * ((4 * dp + 2 * (q & 1) + ((i16 & 3) >> 1)) ^ fs);
  }
  return lo;
}

// o[NRB d + rb]: value columns 128w + 32d .. +31, rows 32rb .. +31 of O^T.
// m_ref, l_part, l_out: the softmax state of this wave's own row
// 32w + lane%32 (both lane halves hold the same values; waves w < NRB).
template <int NRB>
struct R128State {
  f32x16 o[4 * NRB];
  float m_ref, l_part, l_out;
};

// One 32-key tile of bf16 rows in the ring's swizzled layout; the ring
// loads of a later tile are spread over the wave's score MFMAs (issue(m),
// m = 0..8; with LATE, in the 32- and 64-row tiles, from the third one on),
// and side(step, steps) runs once before each of the wave's `steps` score
// MFMAs (the FP8 instance widens the next tile there; with LATE the bf16
// instance resolves the later tile's row addresses in the first two).
template <int NRB, bool LATE = false, class Issue, class Side>
__device__ __forceinline__ void r128_compute(R128State<NRB>& st, const bf16x8 (&qf)[R128_QREG],
                                             const uint8_t* q_tail, const uint8_t* stage, uint8_t* p_lds,
                                             float* alpha_lds, float scale_log2, int ts, int k1, int nrow, int kfull,
                                             int lane, int wave, Issue&& issue, const R128LaneOff& lo,
                                             uint8_t* xchg, Side&& side) {
  const int r = lane & 31, h = lane >> 5;
  if constexpr (NRB < 4) {
    // 32- and 64-row tiles: the score MFMAs of row block rb are split across
    // the DS = 4/NRB waves rb + NRB*s by dims (wave slice s: k-steps
    // s*KS .. s*KS + KS-1), the slices s > 0 hand their partial S^T to the
    // slice-0 wave through LDS, which adds them in slice order and runs the
    // softmax of the block's rows
    constexpr int DS = 4 / NRB, KS = 36 / DS;
    const int slice = wave / NRB;
    f32x16 sc = {};
    bf16x8 kf[4];
    auto k_at = [&](int j) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(stage + lo.k[j & 3] + 128 * (j >> 2));
    };
#pragma unroll
    for (int j = 0; j < 3; ++j) kf[j] = k_at(j);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      if (j + 3 < KS) kf[(j + 3) % 4] = k_at(j + 3);
      // the wave's ring loads of a later tile, spread over its MFMAs
      constexpr int NL = RING_DMA_PER_WAVE;
#pragma unroll
      for (int m = 0; m < NL; ++m)
        if ((LATE ? (m * (KS - 2)) / NL + 2 : (m * KS) / NL) == j) issue(m);
      side(j, KS);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j % 4], qf[j], sc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    f32x16* xw = reinterpret_cast<f32x16*>(xchg) + (size_t)(wave - NRB) * 64 + lane;
    if (slice > 0) *xw = sc;
    __syncthreads();
    if (slice == 0) {
#pragma unroll
      for (int s = 1; s < DS; ++s) sc += reinterpret_cast<const f32x16*>(xchg)[(size_t)(s * NRB + wave - NRB) * 64 + lane];
      float mx = NEG_INF;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = ts + 8 * (i >> 2) + 4 * h + (i & 3);
        sc[i] = (t < k1 && t < nrow) ? sc[i] * scale_log2 : NEG_INF;
        mx = fmaxf(mx, sc[i]);
      }
      float alpha = 1.f;
      if (__ballot(mx > st.m_ref + R128_RESCALE_LOG2) != 0) {
        mx = fmaxf(mx, shfl_xor_fresh(mx, 32));
        if (mx > st.m_ref + R128_RESCALE_LOG2) {
          alpha = fast_exp2(st.m_ref - mx);
          st.l_part *= alpha;
          st.l_out *= alpha;
          st.m_ref = mx;
        }
      }
      const float m_sub = st.m_ref == NEG_INF ? 0.f : st.m_ref;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[i] = fast_exp2(sc[i] - m_sub);
        st.l_part += sc[i];
      }
      uint8_t* prow = p_lds + (32 * wave + r) * R128_PROW + 8 * h;
      bf16x4 p4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        p4[q] = to_bf16x4(sc[4 * q + 0], sc[4 * q + 1], sc[4 * q + 2], sc[4 * q + 3]);
        *reinterpret_cast<bf16x4*>(prow + 16 * q) = p4[q];
      }
      st.l_out = sum_bf16x8(__builtin_shufflevector(p4[0], p4[1], 0, 1, 2, 3, 4, 5, 6, 7), st.l_out);
      st.l_out = sum_bf16x8(__builtin_shufflevector(p4[2], p4[3], 0, 1, 2, 3, 4, 5, 6, 7), st.l_out);
      if (h == 0) alpha_lds[32 * wave + r] = alpha;
    }
  } else {
  // ---- scores of this wave's rows: S^T[key][row], lane holds keys
  // 8*(i/4) + 4h + i%4 of row r
  f32x16 sc = {};
  const uint8_t* kp[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) kp[b] = stage + lo.k[b];
  // K fragments (and the last k-steps of Q^T, from this wave's LDS copy laid
  // out [kk][lane]) are read three k-steps ahead of their MFMA
  bf16x8 kf[4], qt[4];
  auto q_at = [&](int kk) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(q_tail + ((kk - R128_QREG) * 64 + lane) * 16);
  };
#pragma unroll
  for (int kk = 0; kk < 3; ++kk) {
    kf[kk] = *reinterpret_cast<const bf16x8*>(kp[kk & 3] + 128 * (kk >> 2));
    if (kk >= R128_QREG) qt[kk % 4] = q_at(kk);
  }
#pragma unroll
  for (int kk = 0; kk < 36; ++kk) {
    if (kk + 3 < 36) {
      kf[(kk + 3) % 4] = *reinterpret_cast<const bf16x8*>(kp[(kk + 3) & 3] + 128 * ((kk + 3) >> 2));
      if (kk + 3 >= R128_QREG) qt[(kk + 3) % 4] = q_at(kk + 3);
    }
    if ((kk & 3) == 0) issue(kk >> 2);
    side(kk, 36);
    const bf16x8 qv = kk < R128_QREG ? qf[kk < R128_QREG ? kk : 0] : qt[kk % 4];
    const bf16x8 kv = kf[kk % 4];
    // the score accumulator in VGPRs (the builtin puts it in AGPRs, where
    // the allocator then moves a block of O out and back every tile)
    if (kk == 0)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(sc) : "v"(kv), "v"(qv));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sc) : "v"(kv), "v"(qv));
    // keep each step's reads three steps ahead of their MFMA (the scheduler
    // would otherwise sink them next to their use)
    __builtin_amdgcn_sched_barrier(0);
  }
  // the compiler's hazard checker does not see into the asm: the wait states
  // the ISA requires between an MFMA's write of VGPRs and VALU reads of
  // them, with room to spare (24; chained MFMAs accumulating in place need
  // none)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(sc));
  // ---- online softmax of the wave's rows (keys past the piece or past a
  // row's bound masked; tiles below kfull, the wave's smallest bound, need
  // no mask)
  float mx = NEG_INF;
  if (ts + R128_TILE <= kfull) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] *= scale_log2;
      mx = fmaxf(mx, sc[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = ts + 8 * (i >> 2) + 4 * h + (i & 3);
      sc[i] = (t < k1 && t < nrow) ? sc[i] * scale_log2 : NEG_INF;
      mx = fmaxf(mx, sc[i]);
    }
  }
  float alpha = 1.f;
  if (__ballot(mx > st.m_ref + R128_RESCALE_LOG2) != 0) {
    mx = fmaxf(mx, shfl_xor_fresh(mx, 32));
    if (mx > st.m_ref + R128_RESCALE_LOG2) {
      alpha = fast_exp2(st.m_ref - mx);
      st.l_part *= alpha;
      st.l_out *= alpha;
      st.m_ref = mx;
    }
  }
  // masked scores are -inf and exp2(-inf) = 0; a row with no visible key
  // yet has only -inf scores and a -inf reference, so it subtracts 0
  const float m_sub = st.m_ref == NEG_INF ? 0.f : st.m_ref;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sc[i] = fast_exp2(sc[i] - m_sub);
    st.l_part += sc[i];
  }
  // P (bf16) of row 32w + r, keys 8q + 4h .. +3 for q = 0..3, into the
  // workgroup's [128 rows][32 keys] tile; the row's rescale factor beside it
  uint8_t* prow = p_lds + (32 * wave + r) * R128_PROW + 8 * h;
  bf16x4 p4[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    p4[q] = to_bf16x4(sc[4 * q + 0], sc[4 * q + 1], sc[4 * q + 2], sc[4 * q + 3]);
    *reinterpret_cast<bf16x4*>(prow + 16 * q) = p4[q];
  }
  st.l_out = sum_bf16x8(__builtin_shufflevector(p4[0], p4[1], 0, 1, 2, 3, 4, 5, 6, 7), st.l_out);
  st.l_out = sum_bf16x8(__builtin_shufflevector(p4[2], p4[3], 0, 1, 2, 3, 4, 5, 6, 7), st.l_out);
  if (h == 0) alpha_lds[32 * wave + r] = alpha;
  }
  __syncthreads();
  // O^T[dv][row] += V^T[dv][key] P^T[key][row] over 2 k-steps of 16 keys:
  // contraction slot 8h + s is key 16ks + 8h + s on both sides.
  //   B (P^T): lane reads keys 16ks + 8h .. +7 of row 32rb + r (16 bytes).
  //   A (V^T): two transposed reads, keys 16ks + 8h + 4rd + (i16/4), value
  //   columns 32D + 16(q%2) + 4(i16%4) .. +3 for D = 4w + d (q = lane/16,
  //   i16 = lane%16): logical chunk 4D + 2(q%2) + (i16%4)/2, byte 8(i16%2).
  const uint8_t* vp[2][2];  // [rd][d%2]
#pragma unroll
  for (int rd = 0; rd < 2; ++rd)
#pragma unroll
    for (int dp = 0; dp < 2; ++dp) vp[rd][dp] = stage + lo.v[rd][dp];
  const uint8_t* pb = p_lds + r * R128_PROW + 16 * h;
  bf16x8 bp[2][NRB];
  i16x4 v[2][4][2];
  auto pv_operands = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) bp[ks][rb] = *reinterpret_cast<const bf16x8*>(pb + 32 * rb * R128_PROW + 32 * ks);
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd)
        v[ks][d][rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vp[rd][d & 1] + 16 * ks * R128_ROWB + 128 * (d >> 1)));
  };
  // the first k-step's operands are read before the rescale check, so their
  // LDS latency overlaps it
  pv_operands(0);
  // ---- this wave's value columns for all 128 rows.  The accumulator
  // column of lane l is row 32rb + l%32 in block rb: rescale the blocks whose
  // rows moved their reference (rare)
  float ab[NRB];
  bool moved = false;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    ab[rb] = alpha_lds[32 * rb + r];
    moved = moved || ab[rb] != 1.f;
  }
  if (__ballot(moved) != 0) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // in place on the accumulator register (a plain multiply makes the
          // register allocator keep two copies of all 256 accumulators)
          float tmp;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(st.o[NRB * d + rb][i]), "=&v"(tmp) : "v"(ab[rb]));
        }
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks > 0) pv_operands(ks);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x8 av = __builtin_shufflevector(__builtin_bit_cast(bf16x4, v[ks][d][0]),
                                                __builtin_bit_cast(bf16x4, v[ks][d][1]), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        st.o[NRB * d + rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bp[ks][rb], st.o[NRB * d + rb], 0, 0, 0);
    }
  }
}

// The partial slot of one 128-row piece (every wave calls it with its own
// O^T quarter and row state; sums_lds is 128 floats of LDS that no wave still
// reads).
template <int NRB>
__device__ __forceinline__ void r128_store_slot(const DecodeArgs& a, const R128State<NRB>& st, int64_t slot_idx,
                                                float* sums_lds, int wave, int lane) {
  constexpr int ROWS = 32 * NRB;
  // partial slot: O^T / (the row's bf16 sum of P) in fp16, in the
  // accumulator layout [dv/32][row][h][i] (the 16 values a lane holds per
  // 32x32 block are contiguous: 2 x 16-byte stores), then per row m, the
  // fp32 and the bf16 sums of P, then per (value-column quarter, row) the
  // power of two the quarter's fp16 values are to be multiplied by.  The
  // quotients are bounded by the largest |V| of the piece, which can be
  // any bf16 magnitude: each wave scales its 128 columns of a row so that
  // their largest magnitude lies in [2^14, 2^15), inside fp16's range and
  // above its subnormals.  The accumulator columns span all 128 rows,
  // whose sums the owning waves publish through LDS.
  const float l_row = st.l_part + shfl_xor_fresh(st.l_part, 32);
  const float lo_row = st.l_out + shfl_xor_fresh(st.l_out, 32);
  uint8_t* slot = reinterpret_cast<uint8_t*>(a.partials) + slot_idx * r128_slot_bytes(ROWS);
  float* pm = reinterpret_cast<float*>(slot + r128_o_bytes(ROWS));
  const int r = lane & 31, h = lane >> 5;
  if (h == 0 && wave < NRB) sums_lds[32 * wave + r] = lo_row;
  __syncthreads();
  float inv[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float lo = sums_lds[32 * rb + r];
    inv[rb] = lo > 0.f ? 1.f / lo : 0.f;
    // the row's largest quotient over this wave's 128 columns (both lane
    // halves), and the power of two that brings it into [2^14, 2^15)
    float mx = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(st.o[NRB * d + rb][i]));
    mx *= inv[rb];
    mx = fmaxf(mx, shfl_xor_fresh(mx, 32));
    int e = 0;
    if (mx > 0.f && mx <= 3.0e38f) {
      frexpf(mx, &e);  // mx < 2^e
      e = e < -100 ? -100 : e;
    } else {
      e = 15;  // zero, or not finite: factor 1
    }
    inv[rb] *= __builtin_ldexpf(1.f, 15 - e);
    if (h == 0) pm[3 * ROWS + wave * ROWS + 32 * rb + r] = __builtin_ldexpf(1.f, e - 15);
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      _Float16* pl = reinterpret_cast<_Float16*>(slot) + ((4 * wave + d) * ROWS + 32 * rb + r) * 32 + h * 16;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (_Float16)(st.o[NRB * d + rb][8 * c + e] * inv[rb]);
        *reinterpret_cast<f16x8*>(pl + 8 * c) = v;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  if (h == 0 && wave < NRB) {
    const int prow = wave * 32 + r;
    pm[prow] = st.m_ref;
    pm[ROWS + prow] = l_row;
    pm[2 * ROWS + prow] = lo_row;
  }
}

template <bool F8, int NRB>
__global__ __launch_bounds__(R128_THREADS, 1) void attn_r128_kernel(DecodeArgs a) {
  constexpr int ROWS = 32 * NRB;
  // FP8 cache: two stages of 18 KiB (32 rows of 576 E4M3 bytes) and two
  // bf16 tiles `wide` (as much LDS as the bf16 ring): while tile it is
  // computed from one bf16 tile, tile it+1 is widened into the other and
  // tile it+2 loads into the E4M3 stage tile it came from
  constexpr int STAGE = F8 ? M16F8_RAW : R128_STAGE;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[(F8 ? 2 : R128_NS) * STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t wide[F8 ? 2 * R128_STAGE : 16];
  __shared__ int bt_lds[R128_BT_WIN];
  // the 128-row tile keeps Q^T's last k-steps here; smaller tiles exchange
  // partial scores between the waves of a row block here instead
  __shared__ __attribute__((aligned(16)))
  uint8_t q_tail_lds[NRB == 4 ? 4 * R128_QLDS * 64 * 16 : (4 - NRB) * 64 * 64];
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[ROWS * R128_PROW];
  __shared__ float alpha_lds[ROWS];
  __shared__ PlanLds<R128_THREADS> plan;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // 128-row tiles keep a bundle's workgroups on one XCD; smaller tiles
  // (one per request) take ranges in launch order, as the 16-row kernel does
  const int w = (NRB == 4 || a.n_rt > 1 || a.vrt) ? xcd_range_index(blockIdx.x, a.G) : (int)blockIdx.x;
  const int bund = w / a.n_rt, tile = w - bund * a.n_rt;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)ring;
  int dma_sel_off[RING_DMA_PER_WAVE];  // per-lane constants of this wave's ring loads
  ring_dma_offsets(dma_sel_off, wave, lane);
  // the wave's row block and, for tiles under 128 rows, its slice of the dims
  const int wrb = NRB == 4 ? wave : wave % NRB;
  const int wkb0 = NRB == 4 ? 0 : (wave / NRB) * (36 / (4 / NRB));
  const R128LaneOff lane_off = r128_lane_offsets(lane, wave, wkb0);

  for_each_piece<R128_THREADS>(a, bund, tile, plan, [&](int bb, int rt, int k0, int k1, int seq, int tot) {
    // ---- one piece: rows [128 rt, 128 rt + 128) of request bb, keys [k0, k1);
    // a row tile past the request's rows (a shorter query in a varlen
    // batch) has nothing to compute
    int q_len, q_base;
    request_tokens(a, bb, q_len, q_base);
    q_len = __builtin_amdgcn_readfirstlane(q_len);
    q_base = __builtin_amdgcn_readfirstlane(q_base);
    if (rt * ROWS >= q_len * a.H) return;
    const int32_t* btr = a.bt + (int64_t)bb * a.max_blocks;
    const int lf = lane_id_fresh();
    const int row0 = rt * ROWS + wave * 32;  // the wave's first row
    const int my_row = row0 + (lf & 31);
    const bool row_ok = wave < NRB && my_row < q_len * a.H;
    const int nrow = row_ok ? row_bound(seq, tot, q_len, my_row / a.H, a.W, a.rank, a.I, a.causal) : 0;
    // the smallest bound over the wave's rows (tiles below it are unmasked):
    // a row's bound grows with its query token, so it is the first row's
    // bound, or 0 when a row of the wave lies past the request's rows
    int nmin = 0;
    if (wave < NRB && row0 + 31 < q_len * a.H) nmin = row_bound(seq, tot, q_len, row0 / a.H, a.W, a.rank, a.I, a.causal);
    nmin = __builtin_amdgcn_readfirstlane(nmin);
    bf16x8 qf[R128_QREG];
    uint8_t* q_tail = q_tail_lds + (NRB == 4 ? wave * R128_QLDS * 64 * 16 : 0);
    if constexpr (!F8) {
      // the tile's query rows come through the ring like key tiles (32 rows
      // per stage, 1 KiB contiguous loads, rows past the request's rows
      // read the zero row): row blocks 0 .. 2 into stages 0 .. 2, then row
      // block 3 into stage 0.  Each wave reads its fragments from its row
      // block's stage in the key fragments' layout (k-step kb0 + j at
      // lane_off.k[j % 4] + 128 (j / 4)).  The previous piece's waves are
      // all past their last ring read (the barrier before its slot store).
      const R128LaneOff qlo = r128_lane_offsets(lf, wave, wkb0);
      auto q_rows = [&](int rb, uint32_t stage_lds) __attribute__((always_inline)) {
        const int row = rt * ROWS + 32 * rb + 8 * wave + (lf & 7);
        const uint8_t* rowp = reinterpret_cast<const uint8_t*>(kZeroRow);
        asm volatile("" : "+v"(rowp));
        if (row < q_len * a.H) rowp = a.q + ((int64_t)q_base * a.H + row) * ROW_BYTES;
        return ring_rows(rowp, stage_lds);
      };
      auto q_frags = [&](const uint8_t* stage) __attribute__((always_inline)) {
        if constexpr (NRB == 4) {
#pragma unroll
          for (int kk = 0; kk < R128_QREG; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8*>(stage + qlo.k[kk & 3] + 128 * (kk >> 2));
#pragma unroll
          for (int kk = R128_QREG; kk < 36; ++kk)
            *reinterpret_cast<bf16x8*>(q_tail + ((kk - R128_QREG) * 64 + lf) * 16) =
                *reinterpret_cast<const bf16x8*>(stage + qlo.k[kk & 3] + 128 * (kk >> 2));
        } else {
          constexpr int KS = 36 / (4 / NRB);
#pragma unroll
          for (int j = 0; j < KS; ++j)
            qf[j] = *reinterpret_cast<const bf16x8*>(stage + qlo.k[j & 3] + 128 * (j >> 2));
        }
      };
      constexpr int R1 = NRB < 3 ? NRB : 3;
#pragma unroll
      for (int rb = 0; rb < R1; ++rb) ring_issue_all(q_rows(rb, ring_lds + rb * STAGE), wave, dma_sel_off);
      WAIT_VMCNT(0);
      __syncthreads();
      if (wrb < R1) q_frags(ring + wrb * STAGE);
      if constexpr (NRB == 4) {
        __syncthreads();
        ring_issue_all(q_rows(3, ring_lds), wave, dma_sel_off);
        WAIT_VMCNT(0);
        __syncthreads();
        if (wave == 3) q_frags(ring);
      }
      // the sub-piece loop's first barrier orders these reads before the
      // prologue's loads into stage 0
    } else if constexpr (NRB == 4) {
      const uint8_t* qrow = a.q + ((int64_t)q_base * a.H + (row_ok ? my_row : 0)) * ROW_BYTES + 16 * (lane >> 5);
#pragma unroll
      for (int kk = 0; kk < R128_QREG; ++kk) qf[kk] = row_ok ? gload_bf16x8(qrow + 32 * kk) : zero_bf16x8();
#pragma unroll
      for (int kk = 0; kk < R128_QLDS; ++kk)
        *reinterpret_cast<bf16x8*>(q_tail + (kk * 64 + lane) * 16) =
            row_ok ? gload_bf16x8(qrow + 32 * (R128_QREG + kk)) : zero_bf16x8();
    } else {
      // this wave's slice of the dims of its row block's query rows
      constexpr int KS = 36 / (4 / NRB);
      const int qr = rt * ROWS + wrb * 32 + (lane & 31);
      const bool q_ok = qr < q_len * a.H;
      const uint8_t* qrow = a.q + ((int64_t)q_base * a.H + (q_ok ? qr : 0)) * ROW_BYTES + 16 * (lane >> 5) + 32 * wkb0;
#pragma unroll
      for (int j = 0; j < KS; ++j) qf[j] = q_ok ? gload_bf16x8(qrow + 32 * j) : zero_bf16x8();
    }
    R128State<NRB> st;
#pragma unroll
    for (int m = 0; m < 4 * NRB; ++m) st.o[m] = f32x16{};
    st.m_ref = NEG_INF;
    st.l_part = 0.f;
    st.l_out = 0.f;

    // sub-pieces whose block-table span fits the LDS window
    const int span_keys = (R128_BT_WIN - 1) * a.bs;
    for (int ka = k0; ka < k1; ka += span_keys) {
      const int kb = (k1 - ka) < span_keys ? k1 : ka + span_keys;
      const int e0 = block_of(a, ka), e1 = block_of(a, kb - 1);
      __syncthreads();  // previous sub-piece done with the window and the ring
      for (int e = e0 + tid; e <= e1; e += R128_THREADS) bt_lds[e - e0] = e < a.max_blocks ? gload_i32(btr + e) : -1;
      __syncthreads();
      const int nt = (kb - ka + R128_TILE - 1) / R128_TILE;
      if constexpr (F8) {
        // E4M3 tile t lands in stage t%2 and is widened into bf16 tile t%2
        // while tile t-1 is computed.  Loads go out spread over the score
        // MFMAs, or (blocks under 32 keys, a row lookup per lane) together.
        auto issue_tile = [&](const F8Tile& T) __attribute__((always_inline)) {
#pragma unroll
          for (int m = 0; m < 5; ++m) {
            if (T.rowwise)
              r128f8_issue_rowwise(a, bt_lds, e0, T, m, wave);
            else
              r128f8_issue(T, m, wave, lane);
          }
        };
        issue_tile(r128f8_tile(a, bt_lds, e0, ka, kb, ring_lds));
        issue_tile(r128f8_tile(a, bt_lds, e0, ka + R128_TILE, kb, ring_lds + STAGE));
        if (wave < 2)
          WAIT_VMCNT(5);  // tile 0 landed; tile 1's five loads may stay in flight
        else
          WAIT_VMCNT(4);
        __syncthreads();
        r128f8_widen(ring, wide, wave, lane);
        for (int it = 0; it < nt; ++it) {
          const uint32_t par = it & 1;
          // tile it+1 landed (its loads were the only ones in flight), and
          // every wave is done with bf16 tile it-1 and with E4M3 tile it ...
          WAIT_VMCNT(0);
          __syncthreads();
          // ... so bf16 tile it is whole, tile it+1 can be widened into
          // bf16 tile it-1's place and tile it+2 loaded into E4M3 tile it's
          const F8Tile nxt8 = r128f8_tile(a, bt_lds, e0, ka + (it + 2) * R128_TILE, kb, ring_lds + par * STAGE);
          if (nxt8.rowwise) issue_tile(nxt8);
          const uint8_t* s_nxt = ring + (par ^ 1) * STAGE;
          uint8_t* w_nxt = wide + (par ^ 1) * R128_STAGE;
          uint2 pend = {0u, 0u};
          r128_compute<NRB>(
              st, qf, q_tail, wide + par * R128_STAGE, p_lds, alpha_lds, a.scale_log2, ka + it * R128_TILE, kb, nrow,
              min(kb, nmin), lane, wave,
              [&](int m) __attribute__((always_inline)) {
                if (m < 5 && !nxt8.rowwise) r128f8_issue(nxt8, m, wave, lane);
              },
              lane_off, q_tail_lds,
              // item i read at step i*steps/9 and written steps/18 steps later
              [&](int step, int steps) __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < 9; ++i) {
                  const int rs = (i * steps) / 9, ws = rs + (steps >= 18 ? steps / 18 : 0);
                  if (step == rs) pend = r128f8_widen_read(s_nxt, wave, lane, i);
                  if (step == ws) r128f8_widen_write(w_nxt, wave, lane, i, pend);
                }
              });
        }
      } else {
        // prologue: tiles 0 and 1
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const RingRows rr = r128_tile_rows(a, bt_lds, e0, ka + p * R128_TILE, kb, ring_lds + p * STAGE, wave, lane);
          ring_issue_all(rr, wave, dma_sel_off);
        }
        // stage offsets of tiles it and it+2, rotated instead of computed
        // from it % 3 (which costs every LDS address extra instructions)
        uint32_t cur = 0, nxt_off = 2 * STAGE;
        // 128-row tile: the block-table entry of the tile loaded next, read
        // one tile ahead (the same value in every lane)
        int bt_ahead = -1;
        if (NRB == 4 && a.kalign == 32 && ka + 2 * R128_TILE < kb) bt_ahead = bt_lds[block_of(a, ka + 2 * R128_TILE) - e0];
        for (int it = 0; it < nt; ++it) {
          // tile it landed (only tile it+1's 9 loads may still be in flight),
          // then every wave is also done with tile it-1 (its stage and the P
          // tile), so its stage can take tile it+2, loaded while tile it is
          // computed
          WAIT_VMCNT(R128_DMA_PER_WAVE);
          __syncthreads();
          if constexpr (NRB < 4) {
            // tile it+2's row addresses: the block-table read is issued
            // before the first score MFMA and used after it, so its latency
            // and the address arithmetic run under the MFMAs; the tile's
            // loads start at the third k-step.  (The 128-row tile, with four
            // times the MFMAs per tile, gains nothing from this.)
            RingRows nxt;
            int nt_t = 0, nt_blk = -1;
            r128_compute<NRB, true>(
                st, qf, q_tail, ring + cur, p_lds, alpha_lds, a.scale_log2, ka + it * R128_TILE, kb, nrow,
                min(kb, nmin), lane, wave,
                [&](int m) __attribute__((always_inline)) { ring_issue_one(nxt, m, wave, dma_sel_off); }, lane_off,
                q_tail_lds, [&](int step, int) __attribute__((always_inline)) {
                  if (step == 0) {
                    nt_t = ka + (it + 2) * R128_TILE + 8 * wave + (lane_id_fresh() & 7);
                    if (nt_t < kb) nt_blk = bt_lds[block_of(a, nt_t) - e0];
                  } else if (step == 1) {
                    const uint8_t* rowp = reinterpret_cast<const uint8_t*>(kZeroRow);
                    asm volatile("" : "+v"(rowp));
                    if (nt_t < kb && (unsigned)nt_blk < (unsigned)a.num_blocks) {
                      const int vb = block_of(a, nt_t);
                      rowp = a.kv + ((int64_t)nt_blk * a.bs + (nt_t - vb * a.bs)) * ROW_BYTES;
                    }
                    nxt = ring_rows(rowp, ring_lds + nxt_off);
                  }
                });
          } else {
            // tile it+2 on a 32-key boundary lies in one block when 32
            // divides the block size: its 32 rows are contiguous, one
            // block-table entry (read a tile ahead) gives all the wave's row
            // addresses in scalar arithmetic.  Other tiles (a piece's last,
            // or an invalid block id) resolve their rows lane by lane.
            const int ts2 = ka + (it + 2) * R128_TILE;
            const int blk2 = __builtin_amdgcn_readfirstlane(bt_ahead);
            if (a.kalign == 32 && ts2 + R128_TILE < kb) bt_ahead = bt_lds[block_of(a, ts2 + R128_TILE) - e0];
            RingRows nxt;
            if (a.kalign == 32 && ts2 + R128_TILE <= kb && (ts2 & 31) == 0 && (unsigned)blk2 < (unsigned)a.num_blocks) {
              const int vb = block_of(a, ts2);
              const uint64_t r0 = reinterpret_cast<uint64_t>(a.kv) +
                                  (uint64_t)((int64_t)blk2 * a.bs + (ts2 - vb * a.bs) + 8 * wave) * ROW_BYTES;
#pragma unroll
              for (int k = 0; k < 8; ++k) nxt.rows[k] = r0 + (uint64_t)k * ROW_BYTES;
              nxt.stage_lds = ring_lds + nxt_off;
            } else {
              nxt = r128_tile_rows(a, bt_lds, e0, ts2, kb, ring_lds + nxt_off, wave, lane);
            }
            r128_compute<NRB>(st, qf, q_tail, ring + cur, p_lds, alpha_lds, a.scale_log2, ka + it * R128_TILE, kb,
                              nrow, min(kb, nmin), lane, wave,
                              [&](int m) __attribute__((always_inline)) { ring_issue_one(nxt, m, wave, dma_sel_off); },
                              lane_off, q_tail_lds, [](int, int) {});
          }
          nxt_off = cur;
          cur = __builtin_amdgcn_readfirstlane(cur == (R128_NS - 1) * STAGE ? 0u : cur + STAGE);
        }
      }
      WAIT_VMCNT(0);
    }
    __syncthreads();  // every wave is past its last read of alpha_lds
    r128_store_slot(a, st, piece_slot(a, bund, bb, rt), alpha_lds, wave, lane);
  });
}

// ---------------------------------------------------------------- combine
// Grid: (request, row tile) groups x 8 slices of 64 output columns.  Merges
// the partial slots of the workgroups that covered the group and writes bf16
// out and (slice 0) the LSE.  Groups no workgroup covered (no visible keys)
// get out = 0, lse = -inf.
// Partial slot element (row, dv): both kernels store their MFMA accumulator
// layouts.  M16: [dv/16][g][row][i] with dv % 16 = 4g + i; R128:
// [dv/32][row][h][i] with dv % 32 = 8*(i/4) + 4h + i%4.  After the ROWS*512
// values: m[ROWS] (log2 units), the fp32 sums of P[ROWS] (for the LSE) and
// the sums of P as rounded to bf16[ROWS] (for the output); R128 slots then
// hold the fp16 values' factors [4 column quarters][ROWS].
template <int ROWS>
__device__ __forceinline__ int slot_index(int row, int dv) {
  if (ROWS == M16_ROWS) return (dv >> 4) * 256 + ((dv & 15) >> 2) * 64 + row * 4 + (dv & 3);
  const int r32 = dv & 31;
  return ((dv >> 5) * ROWS + row) * 32 + ((r32 >> 2) & 1) * 16 + (r32 >> 3) * 4 + (r32 & 3);
}

// M16 slots hold fp32 O (unnormalised); R128 slots hold fp16 O divided by
// the row's bf16 sum of P and scaled per (column quarter, row) by a power of
// two, so its weight in the merge carries that sum and the factor.
template <int ROWS>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  constexpr int SLICE = 64;                       // output columns per workgroup
  constexpr int PER = ROWS * SLICE / 256;         // outputs per thread
  constexpr bool F16 = ROWS != M16_ROWS;  // slots of the 32-, 64- and 128-row tiles
  constexpr int64_t SLOT_BYTES = F16 ? r128_slot_bytes(ROWS) : (ROWS * D_V + 3 * ROWS) * 4;
  constexpr int O_BYTES = F16 ? r128_o_bytes(ROWS) : ROWS * D_V * 4;
  const int grp = blockIdx.x >> 3, slice = blockIdx.x & 7;
  const int rpt = a.vrt ? a.vrt : a.n_rt;  // row tiles per request
  const int b = grp / rpt, rt = grp - b * rpt;
  const int row = threadIdx.x % ROWS;
  const int col0 = slice * SLICE + (threadIdx.x / ROWS) * PER;
  const int row_idx = rt * ROWS + row;
  int q_len, q_base;
  request_tokens(a, b, q_len, q_base);
  if (row_idx >= q_len * a.H) return;
  // the group's units: its request's (bundles), or its own (per-tile ranges)
  const int64_t T = a.prefix[work_items(a)];
  const int pi = a.vrt ? grp : b;
  const int64_t pb = a.prefix[pi], pb1 = a.prefix[pi + 1];
  const int nb = pb1 > pb ? (int)(pb1 - pb - a.ovh) : 0;
  int j0 = 0, j1 = -1;
  if (nb > 0) {
    // the bundles that hold the request's key units (after its overhead units)
    j0 = range_owner(pb + a.ovh, T, a.nbund, a.wa, a.wb);
    j1 = range_owner(pb + a.ovh + nb - 1, T, a.nbund, a.wa, a.wb);
  }
  const int64_t orow = (int64_t)q_base * a.H + row_idx;
  uint16_t* op = a.out + orow * D_V + col0;
  static_assert(PER % 4 == 0, "outputs are stored 4 columns at a time");
  // bundle j's slot of this group is (j + b) * n_rt + rt = j * n_rt + grp
  // (per-tile ranges: n_rt = 1 and grp is the item, so j + item); a
  // bundle with an empty range wrote nothing.  The slots are merged NMAX at
  // a time: all loads of a batch are issued before any is used.  With at
  // most NMAX slots this is the plain two-pass merge (weights relative to
  // the overall maximum); later batches rescale the running sums.
  constexpr int NMAX = ROWS == M16_ROWS ? 8 : 4;
  // every range holds a unit once T * min(wa, wb) >= Wt
  const bool some_empty = T * (a.wa < a.wb ? a.wa : a.wb) < range_weight(a.nbund, a.nbund, a.wa, a.wb);
  // R128: this thread's columns lie in one 128-column quarter of the slot
  const int quarter = col0 / 128;
  float M = NEG_INF, L = 0.f, Lo = 0.f;
  float acc[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) acc[c] = 0.f;
  for (int jb = j0; jb <= j1; jb += NMAX) {
    float mw[NMAX], lw[NMAX], low[NMAX], fac[NMAX], v[NMAX][PER];
#pragma unroll
    for (int t = 0; t < NMAX; ++t) {
      const int j = jb + t;
      mw[t] = NEG_INF;
      lw[t] = low[t] = 0.f;
      fac[t] = 1.f;
#pragma unroll
      for (int c = 0; c < PER; ++c) v[t][c] = 0.f;
      bool wrote = j <= j1 && (!some_empty || range_nonempty(j, T, a.nbund, a.wa, a.wb));
      if (wrote && a.kalign > 1)  // the piece's keys as request_piece rounds them
        wrote = piece_key(range_start(j + 1, T, a.nbund, a.wa, a.wb) - pb - a.ovh, nb, a.kalign) >
                piece_key(range_start(j, T, a.nbund, a.wa, a.wb) - pb - a.ovh, nb, a.kalign);
      if (wrote) {
        const uint8_t* slot = reinterpret_cast<const uint8_t*>(a.partials) + ((int64_t)j * a.n_rt + grp) * SLOT_BYTES;
        const float* pm = reinterpret_cast<const float*>(slot + O_BYTES);
        mw[t] = pm[row];
        lw[t] = pm[ROWS + row];
        low[t] = pm[2 * ROWS + row];
        if (F16) fac[t] = pm[3 * ROWS + quarter * ROWS + row];
#pragma unroll
        for (int c = 0; c < PER; ++c)
          v[t][c] = F16 ? (float)reinterpret_cast<const _Float16*>(slot)[slot_index<ROWS>(row, col0 + c)]
                        : reinterpret_cast<const float*>(slot)[slot_index<ROWS>(row, col0 + c)];
      }
    }
    float Mb = M;
#pragma unroll
    for (int t = 0; t < NMAX; ++t) Mb = fmaxf(Mb, mw[t]);
    if (Mb == NEG_INF) continue;
    const float sc = (M == NEG_INF) ? 0.f : fast_exp2(M - Mb);
    L *= sc;
    Lo *= sc;
#pragma unroll
    for (int c = 0; c < PER; ++c) acc[c] *= sc;
#pragma unroll
    for (int t = 0; t < NMAX; ++t) {
      const float f = (mw[t] == NEG_INF) ? 0.f : fast_exp2(mw[t] - Mb);
      L += f * lw[t];
      Lo += f * low[t];
      const float fv = F16 ? f * low[t] * fac[t] : f;
#pragma unroll
      for (int c = 0; c < PER; ++c) acc[c] += fv * v[t][c];
    }
    M = Mb;
  }
  if (M == NEG_INF) {
#pragma unroll
    for (int c = 0; c < PER; c += 4) *reinterpret_cast<uint2*>(op + c) = uint2{0u, 0u};
    if (a.lse && slice == 0 && threadIdx.x < ROWS) a.lse[orow] = NEG_INF;
    return;
  }
  const float inv = a.out_scale / Lo;  // the FP8 cache scale of V (1 for bf16)
#pragma unroll
  for (int c0 = 0; c0 < PER; c0 += 4)
    *reinterpret_cast<bf16x4*>(op + c0) = to_bf16x4(acc[c0] * inv, acc[c0 + 1] * inv, acc[c0 + 2] * inv,
                                                     acc[c0 + 3] * inv);
  if (a.lse && slice == 0 && threadIdx.x < ROWS) {
    const float l2 = M + __log2f(L);
    a.lse[orow] = (a.lse_base == MLA_LSE_BASE_E) ? l2 * LN2 : l2;
  }
}

// ---------------------------------------------------------------- host side
struct Plan {
  int rows_tile;
  int n_rt;
  int vrt;
  int ovh;
  int kalign;
  int nbund;
  int wa, wb;  // weights of the first and second half of the ranges
  int G;
  size_t prefix_off, partial_off, bytes;
};

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Requests of up to 16 rows run the 16-row kernel, larger ones the 128-row
// kernel (any block size: a power of two takes shifts, others a division).
Plan make_plan(int B, int q_len, int H, int max_seq_len, int cus, bool fp8 = false, bool varlen = false,
               int block_size = 1) {
  Plan p{};
  const int64_t R = (int64_t)q_len * H;
  p.rows_tile = R <= M16_ROWS ? M16_ROWS : R <= 32 ? 32 : R <= 64 ? 64 : R128_ROWS;
  p.n_rt = (int)((R + p.rows_tile - 1) / p.rows_tile);
  // Per-tile ranges (a query length per request and several row tiles): the
  // (request, row tile) pairs of the requests' actual rows are the work
  // items, laid end to end request by request and cut into one range per
  // workgroup.  Bundles would leave the row-tile workgroups of a shorter
  // request's missing rows idle over its keys.  A request's row tiles are
  // adjacent items, so their ranges mostly fall on one XCD (consecutive
  // workgroup indices) and still share its L2.
  p.vrt = 0;
  if (varlen && p.n_rt > 1 && p.rows_tile != M16_ROWS) {
    p.vrt = p.n_rt;
    p.n_rt = 1;
  }
  // per-group overhead in key units, about what a group's start and end
  // cost in ring time: M16 5 tiles (the query item, a partial tile, the
  // 33 KB partial store and the pipeline refill behind them; 160 units ran
  // about 1% faster than 64, 128, 192 or 256 on the batch-64 single-token
  // workload), 4.5 with an FP8 cache (its tiles carry half the bytes, the
  // query item and the store do not shrink); the larger tiles ~7 tiles
  // (row bounds, query rows, block-table window, ring refill and the
  // partial store: per-workgroup timestamps put a 128-row piece at about
  // 11 us, against 2.1-2.3 us per 32-key tile; 224 ran 2% faster than 96
  // on the DCP-8 shard and 5% on the 16-head spec-decode workload, and as
  // fast as 160 or 288 or faster)
  p.ovh = p.rows_tile == M16_ROWS ? (fp8 ? 144 : 160) : 224;
  // the larger tiles' pieces start on 32-key boundaries when 32 divides the
  // block size: each 32-key tile then lies in one block, and its rows are
  // one contiguous 36 KiB span of the pool
  p.kalign = p.rows_tile != M16_ROWS && block_size % 32 == 0 ? 32 : 1;
  // bundles: balanced key ranges, each processed by n_rt workgroups (one per
  // row tile).  The 128-row kernel keeps a bundle's workgroups on one XCD
  // (8 * k bundles, each XCD holding k whole bundles) so that they share the
  // keys through its L2; a few CUs idle when n_rt does not divide the CUs of
  // an XCD.
  // The 16-row kernel does the same when a request has several row tiles.
  const int per_xcd = (p.rows_tile != M16_ROWS ? 1 : fp8 ? M16F8_WG_PER_CU : 1) * cus / 8;  // resident workgroups
  int64_t nbund = p.n_rt == 1 ? 8 * per_xcd : p.n_rt <= per_xcd ? 8 * (per_xcd / p.n_rt) : 8 * per_xcd / p.n_rt;
  if (nbund < 1) nbund = 1;
  const int64_t units = (int64_t)B * (p.vrt ? p.vrt : 1) * ((max_seq_len > 0 ? max_seq_len : 1) + p.ovh);
  const int64_t by_work = (units + 255) / 256;  // at least 256 keys per workgroup
  if (nbund > by_work) nbund = by_work >= 8 ? by_work / 8 * 8 : by_work;
  if (nbund < 1) nbund = 1;
  p.nbund = (int)nbund;
  p.G = p.nbund * p.n_rt;
  // With two FP8 16-row workgroups on every CU, the first of each pair
  // (launched first, so its waves win issue arbitration) runs its items
  // about 1.2x faster (per-workgroup timestamps on the batch-64
  // single-token workload: 1.79 against 2.14 us per item), and the second
  // half of the workgroups ended 7.5 us later: the first half of the ranges
  // gets 6/5 of the second's share (3% faster than equal shares; 11/10 and
  // 5/4 were in between).
  p.wa = p.wb = 1;
  if (fp8 && p.rows_tile == M16_ROWS && p.nbund == M16F8_WG_PER_CU * cus) {
    p.wa = 6;
    p.wb = 5;
  }
  const size_t slot = p.rows_tile != M16_ROWS ? (size_t)r128_slot_bytes(p.rows_tile)
                                               : (size_t)(p.rows_tile * D_V + 3 * p.rows_tile) * sizeof(float);
  const size_t items = (size_t)B * (p.vrt ? p.vrt : p.n_rt);  // work items; groups of the combine
  p.prefix_off = 0;
  p.partial_off = align_up((size_t)(B * (p.vrt ? p.vrt : 1) + 1) * sizeof(int64_t));
  p.bytes = p.partial_off + align_up(((size_t)p.G + items) * slot);
  return p;
}

thread_local hipEvent_t tl_prof_start = nullptr;
thread_local hipEvent_t tl_prof_stop = nullptr;

}  // namespace

extern "C" int mla_profile_attention_events(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr)) return MLA_ERR_INVALID_ARG;
  tl_prof_start = start;
  tl_prof_stop = stop;
  return MLA_OK;
}

extern "C" size_t mla_decode_workspace_size(int B, int q_len, int H, int max_seq_len) {
  if (B <= 0 || q_len < 1 || H < 1 || max_seq_len < 0) return 0;
  const int cus = device_cu_count();
  size_t m = 0;
  for (const bool fp8 : {false, true})
    for (const bool varlen : {false, true}) {
      const size_t x = make_plan(B, q_len, H, max_seq_len, cus, fp8, varlen).bytes;
      m = x > m ? x : m;
    }
  return m;
}

namespace {

int decode(const void* q, const int32_t* query_start_loc, const void* kv_cache, const int32_t* block_table,
           const int32_t* seq_lens, const int32_t* causal_seqlens_global, int B, int q_len, int H, int num_blocks,
           int block_size,
           int max_blocks, int max_seq_len, int cp_world, int cp_rank, int cp_interleave, int causal, float scale,
           int lse_base, int kv_fp8, float kv_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
           hipStream_t stream) {
  if (B < 0 || q_len < 1 || H < 1 || num_blocks < 1 || block_size < 1 || max_blocks < 1 ||
      max_seq_len < 0 || cp_world < 1 || cp_rank < 0 || cp_rank >= cp_world || cp_interleave < 1 ||
      (int64_t)cp_interleave * cp_world > (1 << 30) ||
      (causal != 0 && causal != 1) || (lse_base != MLA_LSE_BASE_E && lse_base != MLA_LSE_BASE_2) ||
      !std::isfinite(scale) || !(std::isfinite(kv_scale) && kv_scale > 0.f))
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)q_len * H > (1 << 24)) return MLA_ERR_INVALID_ARG;
  if (causal && cp_world > 1 && causal_seqlens_global == nullptr) return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!q || !kv_cache || !block_table || !seq_lens || !out) return MLA_ERR_INVALID_ARG;
  const Plan p = make_plan(B, q_len, H, max_seq_len, device_cu_count(), kv_fp8 != 0, query_start_loc != nullptr,
                           block_size);
  if (workspace_bytes < p.bytes || workspace == nullptr) return MLA_ERR_INVALID_ARG;

  DecodeArgs a{};
  a.q = static_cast<const uint8_t*>(q);
  a.kv = static_cast<const uint8_t*>(kv_cache);
  a.bt = block_table;
  a.seq_lens = seq_lens;
  a.glob = causal_seqlens_global;
  a.qsl = query_start_loc;
  a.B = B; a.Q = q_len; a.H = H; a.R = q_len * H;
  a.num_blocks = num_blocks; a.bs = block_size; a.max_blocks = max_blocks;
  a.bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
  a.W = cp_world; a.rank = cp_rank; a.causal = causal;
  a.I = cp_interleave;
  a.scale_log2 = scale * kv_scale * LOG2E;
  a.out_scale = kv_scale;
  a.kv_fp8 = kv_fp8;
  a.lse_base = lse_base;
  a.n_rt = p.n_rt;
  a.vrt = p.vrt;
  a.rows_tile = p.rows_tile;
  a.ovh = p.ovh;
  a.kalign = p.kalign;
  a.nbund = p.nbund;
  a.wa = p.wa;
  a.wb = p.wb;
  a.G = p.G;
  a.prefix = reinterpret_cast<int64_t*>(static_cast<uint8_t*>(workspace) + p.prefix_off);
  a.partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + p.partial_off);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;

  // the attention kernel; with profiling events set, the runtime records
  // them at the kernel's own start and end (no separate marker packets)
  void (*attn)(DecodeArgs) = nullptr;
  void (*comb)(DecodeArgs) = nullptr;
  switch (p.rows_tile) {
    case M16_ROWS:
      attn = kv_fp8 ? attn_m16_kernel<true> : attn_m16_kernel<false>;
      comb = combine_kernel<M16_ROWS>;
      break;
    case 32:
      attn = kv_fp8 ? attn_r128_kernel<true, 1> : attn_r128_kernel<false, 1>;
      comb = combine_kernel<32>;
      break;
    case 64:
      attn = kv_fp8 ? attn_r128_kernel<true, 2> : attn_r128_kernel<false, 2>;
      comb = combine_kernel<64>;
      break;
    default:
      attn = kv_fp8 ? attn_r128_kernel<true, 4> : attn_r128_kernel<false, 4>;
      comb = combine_kernel<R128_ROWS>;
      break;
  }
  const int threads = p.rows_tile == M16_ROWS ? M16_THREADS : R128_THREADS;
  if (launch(attn, dim3(p.G), dim3(threads), stream, a, tl_prof_start, tl_prof_stop) != hipSuccess)
    return MLA_ERR_HIP;
  if (launch(comb, dim3(B * (p.vrt ? p.vrt : p.n_rt) * 8), dim3(256), stream, a) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

}  // namespace

extern "C" int mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
                          const int32_t* seq_lens, const int32_t* causal_seqlens_global,
                          int B, int q_len, int H, int num_blocks, int block_size, int max_blocks,
                          int max_seq_len, int cp_world, int cp_rank, int causal, float scale,
                          int lse_base, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return decode(q, nullptr, kv_cache, block_table, seq_lens, causal_seqlens_global, B, q_len, H, num_blocks,
                block_size, max_blocks, max_seq_len, cp_world, cp_rank, 1, causal, scale, lse_base, 0, 1.f, out,
                lse, workspace, workspace_bytes, stream);
}

extern "C" int mla_decode_interleaved(const void* q, const void* kv_cache, const int32_t* block_table,
                                      const int32_t* seq_lens, const int32_t* causal_seqlens_global,
                                      int B, int q_len, int H, int num_blocks, int block_size, int max_blocks,
                                      int max_seq_len, int cp_world, int cp_rank, int cp_interleave, int causal,
                                      float scale, int lse_base, void* out, float* lse, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return decode(q, nullptr, kv_cache, block_table, seq_lens, causal_seqlens_global, B, q_len, H, num_blocks,
                block_size, max_blocks, max_seq_len, cp_world, cp_rank, cp_interleave, causal, scale, lse_base, 0,
                1.f, out, lse, workspace, workspace_bytes, stream);
}

extern "C" int mla_decode_varlen(const void* q, const int32_t* query_start_loc, int max_q_len, const void* kv_cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* causal_seqlens_global, int B, int H, int num_blocks, int block_size,
                                 int max_blocks, int max_seq_len, int cp_world, int cp_rank, int cp_interleave,
                                 int causal, float scale, int lse_base, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (B > 0 && query_start_loc == nullptr) return MLA_ERR_INVALID_ARG;
  return decode(q, query_start_loc, kv_cache, block_table, seq_lens, causal_seqlens_global, B, max_q_len, H,
                num_blocks, block_size, max_blocks, max_seq_len, cp_world, cp_rank, cp_interleave, causal, scale,
                lse_base, 0, 1.f, out, lse, workspace, workspace_bytes, stream);
}

extern "C" int mla_decode_fp8(const void* q, const void* kv_cache, float kv_scale, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* causal_seqlens_global, int B, int q_len, int H,
                              int num_blocks, int block_size, int max_blocks, int max_seq_len, int cp_world,
                              int cp_rank, int cp_interleave, int causal, float scale, int lse_base, void* out,
                              float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode(q, nullptr, kv_cache, block_table, seq_lens, causal_seqlens_global, B, q_len, H, num_blocks,
                block_size, max_blocks, max_seq_len, cp_world, cp_rank, cp_interleave, causal, scale, lse_base, 1,
                kv_scale, out, lse, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- no-allocation variant
// mla_decode_noalloc takes its workspace from this array instead of the
// caller.  In host code `scratch` is only a stand-in for the device symbol:
// its device address (one per GPU) comes from hipGetSymbolAddress, looked up
// on the first call on each device with that device current, and only that
// address is passed to kernels.  Nothing in the workspace needs clearing
// between calls: the request offsets are written by the attention kernel
// before the combine reads them, and every partial slot the combine reads
// was written by the same call.
static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's scratch array, or null.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_addr[dev] = ptr;
  }
  return g_scratch_addr[dev];
}

}  // namespace

extern "C" int mla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, const int32_t* causal_seqlens_global, int B, int q_len,
                                  int H, int num_blocks, int block_size, int max_blocks, int max_seq_len,
                                  int cp_world, int cp_rank, int causal, float scale, int lse_base, void* out,
                                  float* lse, hipStream_t stream) {
  if (B < 0 || q_len < 1 || H < 1 || max_seq_len < 0 || (int64_t)q_len * H > (1 << 24)) return MLA_ERR_INVALID_ARG;
  void* ws = nullptr;
  if (B > 0) {
    // sizes beyond the array are refused before anything touches the GPU
    if (make_plan(B, q_len, H, max_seq_len, device_cu_count()).bytes > MLA_NOALLOC_SCRATCH_BYTES)
      return MLA_ERR_INVALID_ARG;
    ws = device_scratch();
    if (ws == nullptr) return MLA_ERR_HIP;
  }
  return decode(q, nullptr, kv_cache, block_table, seq_lens, causal_seqlens_global, B, q_len, H, num_blocks,
                block_size, max_blocks, max_seq_len, cp_world, cp_rank, 1, causal, scale, lse_base, 0, 1.f, out, lse,
                ws, ws ? MLA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
