// Index maps and launch plans of the int8 GEMMs: the prefill kernel's tile
// schedule, K slices, direct-to-LDS transfer addresses, LDS fragment
// offsets, split-K partial-tile offsets and output staging, and the decode
// kernel's step, reduction and partial-tile offsets.
//
// Plain C++ with no HIP types: the kernels call these functions, and a host
// program compiles the same functions to replay every workgroup's and lane's
// addresses against the buffers they must stay inside.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define SQ_HD __host__ __device__ __forceinline__
#else
#define SQ_HD inline
#endif

namespace sqi {

SQ_HD int imin(int a, int b) { return a < b ? a : b; }

// Split-K workspaces (the decode and prefill GEMMs): ticket counters in a
// fixed region at the start, then the partial tiles. The region has room for
// every split the plans below make (the decode kernel splits only below 192
// workgroups, the prefill kernel only below 128 tiles), so the partial tiles
// of one shape never land on the counters of another: one zero-filled
// workspace serves any sequence of calls, of any shapes, made one at a time.
constexpr size_t kSplitCounterBytes = 1024;
constexpr int64_t kSplitMaxCounters = (int64_t)(kSplitCounterBytes / 4);

// ============================================================== prefill ====

constexpr int kBigBM = 256;
constexpr int kBigBK = 128;    // k bytes per pipeline stage: one 128-byte line per tile row
constexpr int kBigStages = 2;  // LDS double buffer
constexpr int kGroupM = 4;
constexpr int kBigMaxSplit = 8;  // at most this many K slices per output tile

// kW waves in a (kW/2) x 2 grid over the 256 x BN tile.
template <int BN, int kW = 8>
struct BigCfg {
  static constexpr int kThreads = 64 * kW;
  static constexpr int kWN = BN / 2;                  // output columns per wave
  static constexpr int kFN = kWN / 32;
  static constexpr int kWM = kBigBM / (kW / 2);        // tokens per wave
  static constexpr int kFM = kWM / 32;
  static constexpr int kStageA = kBigBM * kBigBK;
  static constexpr int kStage = (kBigBM + BN) * kBigBK;
  // 1 KiB direct-to-LDS transfers (8 rows each) per wave and stage
  static constexpr int kDmaA = kBigBM / 8 / kW;
  static constexpr int kDmaB = BN / 8 / kW;
  static constexpr int kDma = kDmaA + kDmaB;
  // split K: one partial tile (int32 or binary32) per slice and tile
  static constexpr uint32_t kTileBytes = kBigBM * BN * 4;
  static constexpr uint32_t kWaveBytes = kTileBytes / kW;
};

// Output tile of workgroup t: workgroups are dispatched round-robin over the
// 8 XCDs, so the first (total & ~7) of them are renumbered to give each XCD a
// contiguous range of tiles; tiles are then visited kGroupM tile-rows at a
// time, column by column, so that tiles sharing Xq and Wq panels run close
// together (under the same L2).
struct BigTile {
  int tm, tn;
};
SQ_HD BigTile big_tile(int t, int nbm, int nbn) {
  const int total = nbm * nbn;
  const int full = total & ~7;
  if (t < full) t = (t & 7) * (full >> 3) + (t >> 3);
  const int in_group = kGroupM * nbn;
  const int first_m = (t / in_group) * kGroupM;
  const int gm = imin(nbm - first_m, kGroupM);
  BigTile r;
  r.tm = first_m + (t % in_group) % gm;
  r.tn = (t % in_group) / gm;
  return r;
}

// K stages [kt0, kt0 + nk) of K slice `slice` (one slice covers all stages
// when the kernel does not split).
struct BigSlice {
  int kt0, nk;
};
SQ_HD BigSlice big_slice(bool split, int slice, int slice_stages, int stages) {
  BigSlice s;
  s.kt0 = split ? slice * slice_stages : 0;
  s.nk = split ? imin(slice_stages, stages - s.kt0) : stages;
  return s;
}

// Byte offset of 16-byte chunk c (0..7) of tile row r in a stage (128-byte
// rows). The chunk index is XOR-ed with (r >> 1) & 7: a 128-byte row covers
// half of the 64 banks, so rows r and r+1 fall in different halves, and the
// eight even (odd) rows of a 16-lane group get eight distinct chunks. Without
// it every lane of a half-wave would hit the same bank group; with r & 7,
// rows r and r + 8 collided (measured: 3.96M bank-conflict cycles per QKV
// dispatch, 0.29M with this one).
SQ_HD int big_swz(int r) { return (r >> 1) & 7; }
SQ_HD int big_lds_off(int r, int c) { return r * kBigBK + ((c ^ big_swz(r)) << 4); }

// Direct-to-LDS transfer i (0 .. kDma-1) of wave `wid`, lane `lane`: lane L
// of a 1 KiB transfer fills LDS bytes [16L, 16L+16) of an 8-row block, i.e.
// row L/8, physical chunk L%8, so it fetches the logical chunk
// (L%8) ^ swizzle(row) of that row; the 8 lanes of a row read one whole
// 128-byte line. `a`: the transfer belongs to the Xq tile (else Wq); `row`:
// tile row; `chunk`: logical 16-byte chunk; `dst`: the block's LDS offset
// within a stage (the lane writes dst + 16 lane).
struct BigDma {
  bool a;
  int row, chunk, dst;
};
template <int BN, int kW>
SQ_HD BigDma big_dma(int i, int wid, int lane) {
  using C = BigCfg<BN, kW>;
  BigDma d;
  d.a = i < C::kDmaA;
  const int blk = (d.a ? i : i - C::kDmaA) * kW + wid;  // 8-row block within the operand tile
  d.row = blk * 8 + (lane >> 3);
  d.chunk = (lane & 7) ^ big_swz(d.row);
  d.dst = (d.a ? 0 : C::kStageA) + blk * 1024;
  return d;
}

// Global byte offset of a transfer's 16 bytes at stage kt: rows past the
// operand's end read its last row (results never stored).
SQ_HD int64_t big_dma_src(int tile_row0, int row, int rows, int K, int kt, int chunk) {
  return (int64_t)imin(tile_row0 + row, rows - 1) * K + (int64_t)kt * kBigBK + chunk * 16;
}

// The same transfers through a buffer resource over the tile's rows of the
// operand (based at row tile_row0, valid_rows = big_tile_rows(...) whole rows
// long): the lane's fixed offset (its row, clamped to the last valid row, and
// chunk) plus the stage's scalar offset, so the loop advances one scalar per
// stage. tile_row0 * K + big_dma_voff(...) + big_dma_soff(kt) equals
// big_dma_src(tile_row0, row, rows, K, kt, chunk).
SQ_HD int big_tile_rows(int tile_row0, int rows, int tile) { return imin(rows - tile_row0, tile); }
SQ_HD int big_dma_voff(int row, int valid_rows, int K, int chunk) { return imin(row, valid_rows - 1) * K + chunk * 16; }
SQ_HD int big_dma_soff(int kt) { return kt * kBigBK; }

// Tile row of fragment i of wave row wm (the lane's row frow = lane % 32).
template <int BN, int kW>
SQ_HD int big_frag_row(int wm, int i, int frow) {
  return wm * BigCfg<BN, kW>::kWM + 32 * i + frow;
}

// Wq tile row (output column) of fragment j of wave column wn.
template <int BN, int kW>
SQ_HD int big_wfrag_row(int wn, int j, int frow) {
  return wn * BigCfg<BN, kW>::kWN + 32 * j + frow;
}

// Tile column of the first of the 4 consecutive outputs that register group
// rg (registers 4 rg .. 4 rg + 3) of a lane's 32x32 accumulator block j
// holds: the block's column 8 rg + 4 (lane / 32) (the lane's token is
// column lane % 32 of the block's transposed product).
template <int BN, int kW>
SQ_HD int big_frag_col(int wn, int j, int rg, int fhalf) {
  return wn * BigCfg<BN, kW>::kWN + 32 * j + 8 * rg + 4 * fhalf;
}

// Split-K partial tiles, kept in accumulator order: slice s, tile t, wave w,
// block q = j * kFM + i, register group rg, lane l at 16 bytes each, so every
// store and load instruction of a wave covers 1 KiB of consecutive bytes.
template <int BN, int kW>
SQ_HD uint32_t big_partial_off(int slice, int total, int tile_id, int wid, int lane, int q, int rg) {
  using C = BigCfg<BN, kW>;
  return ((uint32_t)slice * (uint32_t)total + (uint32_t)tile_id) * C::kTileBytes + (uint32_t)wid * C::kWaveBytes +
         (uint32_t)lane * 16 + (uint32_t)(q * 4 + rg) * 1024;
}

// Output staging of the epilogue (rows of 16-byte-aligned outputs): band
// (i, h) holds fragment row block i of every wave row (kW/2 x 32 tile rows)
// and, when a band of whole rows would not fit one stage buffer, column
// half h. Chunk c of staged row r sits at chunk (c + r) mod kCh.
template <int BN, int kW, int kEl>
struct BigBand {
  static constexpr int kRows = (kW / 2) * 32;  // rows per band
  static constexpr int kParts = kRows * BN * kEl <= BigCfg<BN, kW>::kStage ? 1 : 2;
  static constexpr int kColsB = BN / kParts;  // columns per band
  static constexpr int kRowB = kColsB * kEl;  // staged row bytes
  static constexpr int kCh = kRowB / 16;      // 16-byte chunks per staged row
  static constexpr int kPer = 16 / kEl;       // outputs per chunk
  static_assert(kRows * kRowB <= BigCfg<BN, kW>::kStage, "an output band must fit one stage buffer");
};
SQ_HD int band_chunk(int ch, int lr, int kCh) {
  int pc = ch + lr % kCh;
  if (pc >= kCh) pc -= kCh;
  return pc;
}
// Tile row of staged row lr of band row block i.
template <int BN, int kW>
SQ_HD int band_tile_row(int lr, int i) {
  return (lr >> 5) * BigCfg<BN, kW>::kWM + 32 * i + (lr & 31);
}

// ---- prefill plan (host)

// Whether the 256-row-tile kernel takes this GEMM (split_ok: the call may
// split K, i.e. it is not the LLM.int8() epilogue).
inline bool big_suits(int64_t m, int64_t n, int64_t k, bool split_ok) {
  if (n < 192 || k % kBigBK != 0) return false;
  if (m >= 256 && m * n >= ((int64_t)1 << 20)) return true;
  // 129..255 tokens over wide layers: one 256-row tile per column block with
  // K split over the CUs beats the decode and 128 x 128 kernels (GEMM us at
  // 136 / 192 tokens, decode / 128 x 128 / this: 14336 -> 4096 60.8 / 136.3 /
  // 49.9 and 69.2 / 138.0 / 57.1; 4096 -> 14336 48.9 / 48.6 / 38.0 and 55.4 /
  // 49.8 / 39.1; 4096 -> 28672 91.8 / 60.4 / 47.8 and 110.2 / 61.9 / 53.6),
  // except that the decode kernel streams weights under 32 MiB fast enough to
  // stay ahead up to about 176 tokens (4096 -> 6144: 24.0 / 38.6 / 30.9 at
  // 136 tokens, 36.6 / 39.3 / 31.3 at 192)
  if (!split_ok || n < 4096 || k / kBigBK < 20) return false;
  return m >= 176 || (m >= 129 && n * k >= ((int64_t)1 << 25));
}

struct BigSplit {
  int bn = 256;
  int S = 1;
  int slice_stages = 0;
  int64_t tiles = 0;
};

// K slices for `tiles` output tiles: split when the tiles cover fewer than
// half of the 256 CUs, into at most as many slices as keep all workgroups in
// one wave with a CU to spare (a full 256 measured slower: 4096 -> 6144 at 512
// tokens, 64 tiles in 3 / 4 slices 34.8 / 37.1 us). Each slice costs its
// reducer one more partial tile to read and shortens every slice's main loop:
// with about 1.3 us per 128-deep stage and 3 us per slice (fitted on 14336 ->
// 4096 at 192 tokens: 4 / 8 / 10 slices 56.6 / 49.9 / 52.1 us),
// S = sqrt(0.45 x stages) balances the two (7 for K = 14336, 4 for K = 4096;
// 4096 -> 6144 at 256 tokens: 3 / 4 / 6 slices 32.1 / 31.9 / 34.8 us). Slices
// keep at least 8 stages. A second wave of workgroups costs more than the
// split saves (14336 -> 4096 at 1024 tokens in 3 slices: 112 us against 89 in
// 2), and so does splitting 128 tiles in two (4096 -> 6144 at 1024 tokens:
// 43.2 -> 46.5 us).
inline int big_split_for(int64_t tiles, int stages, int bn) {
  int want = tiles < 128 ? (int)(255 / tiles) : 1;
  int best = (int)(sqrtf(0.45f * (float)stages) + 0.5f);
  if (want > best) want = best;
  if (want > kBigMaxSplit) want = kBigMaxSplit;
  if (want > stages / 8) want = stages / 8;
  if (want < 2) return 1;
  const int per = (stages + want - 1) / want;
  const int S = (stages + per - 1) / per;
  if ((size_t)S * (size_t)tiles * (size_t)(kBigBM * bn * 4) >= ((size_t)1 << 31)) return 1;
  return S;
}

// Tile width (256, 192 or 128 columns) and K split, chosen together: the
// score is the fraction of the scheduled waves' workgroup slots doing useful
// work, useful outputs x S over (waves of tiles x S) x 256 x 256 x BN, times
// a measured efficiency: 0.8 for 128-column tiles (less operand reuse per
// fragment read), 0.8 for a split (0.7 with 256-column tiles). GEMM alone,
// us, tile width 192 / 256 / 128 (S: split into S slices): 4096 -> 6144 at
// 1024 tokens 44.2 / 59.4 (S2) / 36.9; 4096 -> 14336 at 512 tokens 47.8 /
// 63.4 (S2) / 41.6; 14336 -> 4096 at 2048 tokens 134.8 / 146.9 / 126.3, at
// 1024 tokens 97.5 (S2) / 105.9 (S3) / 118.4, at 3072 tokens 269.3 / 167.3 /
// 223.7; 4096 -> 6144 at 1536 tokens 46.2 / 52.9 / 71.0. The 128-column
// tile is taken only unsplit (the combination measured). E4M3 tiles have 192
// or 128 columns.
inline BigSplit big_split(int64_t m, int64_t n, int64_t k, bool f8, bool split_ok) {
  const int stages = (int)(k / kBigBK);
  const int cands[3] = {256, 192, 128};
  BigSplit best;
  double best_score = -1.0;
  for (int bn : cands) {
    if (f8 && bn == 256) continue;
    BigSplit p;
    p.bn = bn;
    p.tiles = ((m + kBigBM - 1) / kBigBM) * ((n + bn - 1) / bn);
    p.S = split_ok ? big_split_for(p.tiles, stages, bn) : 1;
    if (bn == 128 && p.S > 1) continue;
    p.slice_stages = (stages + p.S - 1) / p.S;
    const int64_t waves = (p.tiles * p.S + 255) / 256;
    double score = (double)m * (double)n * p.S / ((double)waves * 256.0 * kBigBM * bn);
    if (bn == 128) score *= 0.8;
    if (p.S > 1) score *= bn == 256 ? 0.7 : 0.8;
    if (score > best_score + 1e-9) {
      best = p;
      best_score = score;
    }
  }
  return best;
}

// Split-K workspace of a prefill plan: the counter region, then S partial
// tiles per output tile (0 when the plan does not split).
inline size_t big_workspace_bytes(const BigSplit& p) {
  if (p.S == 1) return 0;
  return kSplitCounterBytes + (size_t)p.S * (size_t)p.tiles * (size_t)(kBigBM * p.bn * 4);
}

// =============================================================== decode ====

constexpr int kDecRows = 64;    // Wq rows per workgroup
constexpr int kDecStep = 128;   // k bytes per pipeline step
constexpr int kDecWaves = 4;
constexpr int kDecMaxNS = 8;    // most steps per wave (template range)
constexpr int64_t kDecodeMaxM = 256;  // one grid layer per 64 tokens up to here

// Steps [step0, step0 + nsl) of K slice `slice`; nsl >= 1 by construction of
// the plan's slice count.
struct DecSlice {
  int step0, nsl;
};
SQ_HD DecSlice dec_slice(int slice, int slice_steps, int K) {
  DecSlice s;
  s.step0 = slice * slice_steps;
  s.nsl = imin(slice_steps, K / kDecStep - s.step0);
  return s;
}
// Slice step loaded as step i of wave wid: wid + 4 i, or, past the slice end,
// the last step again (valid memory; its product is discarded).
SQ_HD int dec_step(int wid, int i, int nsl) { return imin(wid + kDecWaves * i, nsl - 1); }
SQ_HD bool dec_step_valid(int wid, int i, int nsl) { return wid + kDecWaves * i < nsl; }
// The lane's k bytes of a step: int8, [kb, kb+16) and [kb+64, kb+80); E4M3,
// [kb, kb+32) (two 16-byte loads, the second kHalf = 16 further on).
SQ_HD int dec_kb(bool f8, int lane) { return (f8 ? 32 : 16) * (lane >> 4); }
SQ_HD constexpr int dec_khalf(bool f8) { return f8 ? 16 : 64; }
// Wq row (group g) and Xq row (token block mb) a lane loads; rows past the
// end read the last row (results never stored).
SQ_HD int dec_w_row(int n0, int g, int lane, int N) { return imin(n0 + 16 * g + (lane & 15), N - 1); }
SQ_HD int dec_x_row(int m0, int mb, int lane, int M) { return imin(m0 + 16 * mb + (lane & 15), M - 1); }
// Quad (4 columns) of the reduction buffer row `tok` that holds rows
// 16 g + 4 (lane/16) .. +3 of a wave's 16x16 result: XOR-swizzled by the
// token so that the stores and the row-wise reads are free of bank conflicts.
SQ_HD int dec_red_quad(int g, int lane, int tok) { return (4 * g + (lane >> 4)) ^ (tok & 15); }
// Byte offset of output (m, n) of slice s in the partial tiles [S][M][N].
SQ_HD uint32_t dec_partial_off(int slice, int M, int N, int m, int n) {
  return (uint32_t)((((size_t)slice * M + m) * N + n) * 4);
}

// ---- decode, LDS-ring form (more than 16 tokens)
//
// A workgroup owns 64 rows of Wq and kTok tokens (32 or 64; one grid layer
// per 64 tokens as above) over one K slice. Every 128-byte k-step of both
// tiles is one stage of a ring of kRing LDS buffers, filled by direct-to-LDS
// transfers whose 8 lanes per row fetch whole 128-byte lines (chunks
// swizzled with big_swz, as in the prefill kernel); kRing - 1 stages are in
// flight. The four waves take the four 32-byte k-quarters of every stage
// (one v_mfma_i32_32x32x32_i8 per 32 x 32 block), and their int32 tiles are
// added through LDS at the end, where each thread then owns kSpan
// consecutive outputs of one token.
constexpr int64_t kRingMinTokens = 17;
template <int kTok>
struct RingCfg {
  static constexpr int kRows = kDecRows;
  static constexpr int kStageW = kRows * kDecStep;             // Wq part of a stage
  static constexpr int kStage = (kRows + kTok) * kDecStep;
  static constexpr int kDmaW = kRows / (8 * kDecWaves);        // 1 KiB transfers per wave and stage
  static constexpr int kDmaX = kTok / (8 * kDecWaves);
  static constexpr int kDma = kDmaW + kDmaX;
  static constexpr int kNB = kRows / 32;                       // 32 x 32 blocks per wave
  static constexpr int kMB = kTok / 32;
  static constexpr int kRing = kTok == 64 ? 4 : 6;             // stages in the ring
  static constexpr int kSlots = kNB * kMB * 4 * 64;            // 16-byte accumulator slots per wave
  static constexpr int kRedBytes = kDecWaves * kSlots * 16;
  static constexpr int kSlotsF8 = kMB * 4 * 64;                // E4M3: one Wq block per wave
  static constexpr int kLds = kRing * kStage > kRedBytes ? kRing * kStage : kRedBytes;
  static constexpr int kTpt = 256 / kTok;                      // threads per token in the epilogue
  static constexpr int kSpan = kRows / kTpt;                   // consecutive outputs per thread
  static constexpr int kNG = kSpan / 4;                        // 4-output groups per thread
  static constexpr uint32_t kTileBytes = (uint32_t)kNG * 256 * 16;  // one int32 partial tile
};
// Transfer i (0 .. kDma-1) of wave wid, lane: as big_dma, over the stage's
// 64 Wq rows (w) then its kTok Xq rows.
struct RingDma {
  bool w;
  int row, chunk, dst;
};
template <int kTok>
SQ_HD RingDma ring_dma(int i, int wid, int lane) {
  using C = RingCfg<kTok>;
  RingDma d;
  d.w = i < C::kDmaW;
  const int blk = (d.w ? i : i - C::kDmaW) * kDecWaves + wid;
  d.row = blk * 8 + (lane >> 3);
  d.chunk = (lane & 7) ^ big_swz(d.row);
  d.dst = (d.w ? 0 : C::kStageW) + blk * 1024;
  return d;
}
// LDS offset within a stage of the fragment of block bn (Wq) or bm (Xq) that
// lane reads for k-quarter q (its 16 bytes: chunk 2 q + lane / 32 of row
// lane % 32 of the block).
template <int kTok>
SQ_HD int ring_frag_w(int bn, int q, int lane) {
  return big_lds_off(32 * bn + (lane & 31), 2 * q + (lane >> 5));
}
template <int kTok>
SQ_HD int ring_frag_x(int bm, int q, int lane) {
  return RingCfg<kTok>::kStageW + big_lds_off(32 * bm + (lane & 31), 2 * q + (lane >> 5));
}
// Reduction slot (16 bytes, per wave) of register group rg of block (bn, bm)
// at lane; it holds outputs n = 32 bn + 8 rg + 4 (lane / 32) .. +3 of token
// 32 bm + lane % 32.
template <int kTok>
SQ_HD int ring_slot(int bn, int bm, int rg, int lane) {
  return ((bn * RingCfg<kTok>::kMB + bm) * 4 + rg) * 64 + lane;
}
// Epilogue thread tid: its token within the tile, and the first of the four
// outputs (within the tile's 64) of its group g.
template <int kTok>
SQ_HD int ring_tok(int tid) { return tid / RingCfg<kTok>::kTpt; }
template <int kTok>
SQ_HD int ring_col(int tid, int g) {
  return (tid % RingCfg<kTok>::kTpt) * RingCfg<kTok>::kSpan + 4 * g;
}
// The slot that holds outputs nl .. nl + 3 (nl % 4 == 0) of token ml.
template <int kTok>
SQ_HD int ring_read_slot(int ml, int nl) {
  const int nb = nl & 31;
  return ring_slot<kTok>(nl >> 5, ml >> 5, nb >> 3, 32 * ((nb >> 2) & 1) + (ml & 31));
}
// E4M3 form: wave w takes the 64-byte k-half kh = w & 1 of every stage for
// Wq block bn = w >> 1, one v_mfma_scale_f32_32x32x64_f8f6f4 per token
// block; a lane's 32-byte fragment is chunks 4 kh + 2 (lane / 32) and the
// next one of row lane % 32 of the block (half 0 / 1).
SQ_HD int ring_f8_chunk(int wid, int lane, int half) { return 4 * (wid & 1) + 2 * (lane >> 5) + half; }
template <int kTok>
SQ_HD int ring_f8_frag_w(int wid, int lane, int half) {
  return big_lds_off(32 * (wid >> 1) + (lane & 31), ring_f8_chunk(wid, lane, half));
}
template <int kTok>
SQ_HD int ring_f8_frag_x(int bm, int wid, int lane, int half) {
  return RingCfg<kTok>::kStageW + big_lds_off(32 * bm + (lane & 31), ring_f8_chunk(wid, lane, half));
}
// Reduction slot (per wave) of register group rg of token block bm at lane:
// outputs n = 32 bn + 8 rg + 4 (lane / 32) .. +3 of token 32 bm + lane % 32,
// bn the wave's Wq block. Outputs nl .. nl + 3 of token ml are the sum of
// this slot in waves 2 (nl / 32) and 2 (nl / 32) + 1, in that order.
template <int kTok>
SQ_HD int ring_f8_slot(int bm, int rg, int lane) { return (bm * 4 + rg) * 64 + lane; }
template <int kTok>
SQ_HD int ring_f8_read_slot(int ml, int nl) {
  const int nb = nl & 31;
  return ring_f8_slot<kTok>(ml >> 5, nb >> 3, 32 * ((nb >> 2) & 1) + (ml & 31));
}

// Split K: partial tiles in thread order (slice, counter index ctr, group g,
// thread), 16 bytes each, so that every store and load instruction of a
// wave covers 1 KiB of consecutive bytes; padding rows and tokens travel
// with the rest and never reach y.
SQ_HD uint32_t ring_partial_off(int slice, int nctr, int ctr, int g, int tid, uint32_t tile_bytes) {
  return ((uint32_t)slice * (uint32_t)nctr + (uint32_t)ctr) * tile_bytes + (uint32_t)(g * 256 + tid) * 16;
}

// ---- decode plan (host)

struct DecodePlan {
  int S = 1;
  int slice_steps = 0;
  int ns = 0;      // steps per wave
  int tiles = 0;
  int tb = 1;      // 64-token blocks (grid z)
};

// At least one workgroup per CU (256 CUs), with at most kDecMaxNS steps per
// wave; measured on MI355X, more slices than that only add partial-tile
// traffic and reduction latency. Where the unsplit grid already has 192
// workgroups, three in four of the CUs streaming unsplit K are faster than a
// second round of workgroups (4096 -> 14336, 224 column tiles, GEMM us
// unsplit / 2 slices: M 1 13.8 / 15.0, M 8 13.9 / 16.0, M 32 16.4 / 18.4,
// M 64 20.6 / 27.0).
inline DecodePlan decode_plan(int64_t m, int64_t n, int64_t k) {
  DecodePlan p;
  const int steps = (int)(k / kDecStep);
  p.tiles = (int)((n + kDecRows - 1) / kDecRows);
  p.tb = (int)((m + 63) / 64);
  const int wgs = p.tiles * p.tb;
  int want = (256 + wgs - 1) / wgs;
  if (wgs >= 192) want = 1;
  if (want < 1) want = 1;
  if (want > steps) want = steps;
  int per = (steps + want - 1) / want;
  const int cap = kDecWaves * kDecMaxNS;
  if (per > cap) per = cap;
  p.slice_steps = per;
  p.S = (steps + per - 1) / per;
  // one ticket counter per column tile and token block, in the fixed region;
  // without room for them K is not split, and the slice may then exceed the
  // unrolled kernel's step range (see dec_ring / decode_suits)
  if (p.S > 1 && (int64_t)p.tiles * p.tb > kSplitMaxCounters) {
    p.S = 1;
    p.slice_steps = steps;
  }
  p.ns = (p.slice_steps + kDecWaves - 1) / kDecWaves;
  return p;
}

// Whether the LDS-ring form runs (more than 16 tokens, int8 or E4M3
// operands), and its token tile.
inline bool dec_ring(int64_t m, bool f8) {
  (void)f8;
  return m >= kRingMinTokens;
}
inline int dec_ring_tok(int64_t m) { return m <= 32 ? 32 : 64; }

// Split-K workspace of a decode plan for m x n outputs: the counter region,
// then the partial tiles (0 when not split): [S][m][n] of int32 / binary32
// for the unrolled kernel, S x tiles x tb tiles of 64 x kTok int32 in
// thread order for the ring form.
inline size_t dec_workspace_bytes(const DecodePlan& p, int64_t m, int64_t n, bool ring = false) {
  if (p.S == 1) return 0;
  if (ring)
    return kSplitCounterBytes +
           (size_t)p.S * (size_t)p.tiles * (size_t)p.tb * (size_t)dec_ring_tok(m) * (size_t)kDecRows * 4;
  return kSplitCounterBytes + (size_t)p.S * (size_t)m * (size_t)n * 4;
}

// Whether 65..256 tokens go to the decode kernel rather than the tiled
// kernels. The decode kernel streams Wq once per 64-token layer (time grows
// about linearly with the layers); the tiled kernels are slow when their
// output tiles cover few CUs. Counted in 128 x 128 tile units (a 256 x 192
// prefill tile is 3), decode wins when the tiled kernel has at most 128 units:
// measured on MI355X (GEMM us, tiled -> decode), 4096 -> 14336 columns:
// M 96 42.4 -> 36.0, M 128 43.5 -> 39.8 (decode), M 192 43.3 vs 57.5, M 256
// 43.9 vs 75.0 (tiled); 14336 -> 4096: M 96 113.8 -> 42.7, M 128 125.2 ->
// 47.6, M 192 111.8 -> 68.3 (decode). Where the 256-row prefill kernel
// applies, it splits K over enough workgroups to cover the CUs and beats the
// decode kernel: 14336 -> 4096 at 256 tokens 60.4 us against 89.6, at 192
// tokens 57.1 against 69.2.
inline bool decode_beats_prefill(int64_t m, int64_t n, int64_t k) {
  if (big_suits(m, n, k, true)) return false;
  const int64_t units = ((m + 127) / 128) * ((n + 127) / 128);
  return units <= 128;
}

inline bool decode_suits(int64_t m, int64_t n, int64_t k, bool f8) {
  if (!(m >= 1 && m <= kDecodeMaxM && n >= 1 && n <= INT32_MAX && k % kDecStep == 0)) return false;
  // the partial tiles must fit 32-bit offsets (with the unrolled kernel's
  // eight-slice reducer rounds)
  const DecodePlan p = decode_plan(m, n, k);
  if ((size_t)(p.S + 7) / 8 * 8 * (size_t)m * (size_t)n * 4 >= ((size_t)1 << 31)) return false;
  if (dec_workspace_bytes(p, m, n, true) >= ((size_t)1 << 31)) return false;
  // the unrolled kernel covers at most kDecMaxNS steps per wave (the ring
  // form loops over any slice)
  if (!dec_ring(m, f8) && p.ns > kDecMaxNS) return false;
  if (m <= 64) return true;
  // beyond one 64-token block only where the prefill kernels get few tiles
  return decode_beats_prefill(m, n, k);
}

}  // namespace sqi
