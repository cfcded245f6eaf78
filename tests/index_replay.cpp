// Host replay of the int8 GEMMs' index arithmetic, with bounds checks.
//
// Compiles the same index maps and launch plans the kernels use
// (w8a8_int8_quantization_amd/csrc/gemm_index.hpp) and replays, for every
// template configuration the dispatch can launch and a list of shapes (the
// workloads' own and ragged ones), what each workgroup, wave and lane
// addresses:
//   prefill kernel: tile schedule (a bijection onto the output tiles), K
//     slices (a partition of the K stages), direct-to-LDS transfers (global
//     bytes inside the operands; every LDS byte of a stage written once, and
//     each fragment read finding the row and k chunk it expects), split-K
//     partial tiles (inside the workspace, every 16-byte slot written once
//     per call, 32-bit offsets), the epilogue's LDS staging (each output
//     staged once and copied out from where it was staged) and its global
//     stores (inside y, every output once);
//   decode kernel: K slices and per-wave steps (every step once), operand
//     loads inside the rows, the LDS reduction (each quad read where it was
//     written), partial tiles and the reducer's eight-slice rounds (inside
//     32-bit offsets, reads past the last slice never land inside the
//     buffer), ticket counters inside the fixed region, and the output stores;
//   decode ring form: every LDS byte of a stage written once by the
//     transfers, every fragment read finding its row and k chunk (the four
//     waves' quarters covering each row's eight chunks once), the reduction
//     slots (written once, each output read from the slot that holds it),
//     transfers inside the operands over the whole slice, partial tiles
//     (inside the workspace, every 16-byte slot once per call) and the
//     output stores (every output once).
// Prints "OK <checks>" and exits 0, or prints the first failures and exits 1.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "gemm_index.hpp"

using namespace sqi;

static long long g_checks = 0;
static int g_fail = 0;
static std::string g_ctx;

#define CHECK(cond, ...)                                           \
  do {                                                             \
    ++g_checks;                                                    \
    if (!(cond)) {                                                 \
      if (g_fail < 25) {                                           \
        fprintf(stderr, "FAIL [%s] %s: ", g_ctx.c_str(), #cond);   \
        fprintf(stderr, __VA_ARGS__);                              \
        fprintf(stderr, "\n");                                     \
      }                                                            \
      ++g_fail;                                                    \
    }                                                              \
  } while (0)

// ------------------------------------------------------------------ prefill

// LDS tag of one 16-byte slot of a stage: operand (0 Xq, 1 Wq), tile row and
// logical k chunk.
struct Tag {
  int op = -1, row = -1, chunk = -1;
};

// Checks that depend on the template configuration only (all tiles alike).
template <int BN, int kW, bool kF8>
static void big_config_checks() {
  using C = BigCfg<BN, kW>;
  g_ctx = "big config BN=" + std::to_string(BN) + " kW=" + std::to_string(kW) + (kF8 ? " e4m3" : " int8");
  static_assert(C::kFM * 32 == C::kWM && C::kFN * 32 == C::kWN, "whole 32x32 blocks per wave");
  static_assert(C::kDmaA * 8 * kW == kBigBM && C::kDmaB * 8 * kW == BN, "transfers cover the tiles");
  CHECK(2 * C::kStage <= 160 * 1024, "two stages of %d bytes exceed the 160 KiB LDS", C::kStage);
  // one stage of transfers: every 16-byte slot once, with its tag
  std::vector<Tag> lds(C::kStage / 16);
  std::vector<int> hits(C::kStage / 16, 0);
  for (int wid = 0; wid < kW; ++wid)
    for (int lane = 0; lane < 64; ++lane)
      for (int i = 0; i < C::kDma; ++i) {
        const BigDma d = big_dma<BN, kW>(i, wid, lane);
        const int off = d.dst + 16 * lane;
        CHECK(d.dst % 1024 == 0, "transfer block at %d", d.dst);
        CHECK(off >= (d.a ? 0 : C::kStageA) && off + 16 <= (d.a ? C::kStageA : C::kStage), "lds off %d (a=%d)", off,
              (int)d.a);
        CHECK(d.row >= 0 && d.row < (d.a ? kBigBM : BN), "row %d", d.row);
        CHECK(d.chunk >= 0 && d.chunk < 8, "chunk %d", d.chunk);
        if (off < 0 || off + 16 > C::kStage) continue;
        // the physical slot the lane fills is the one the fragment map assigns
        // to (row, chunk)
        CHECK((d.a ? 0 : C::kStageA) + big_lds_off(d.row, d.chunk) == off, "slot %d vs map %d", off,
              big_lds_off(d.row, d.chunk));
        ++hits[off / 16];
        lds[off / 16] = Tag{d.a ? 0 : 1, d.row, d.chunk};
      }
  for (size_t s = 0; s < hits.size(); ++s) CHECK(hits[s] == 1, "LDS slot %zu written %d times", s, hits[s]);
  // fragment reads: each 16-byte read finds (operand, row, chunk) it expects,
  // and over a stage's substeps a lane pair (l, l + 32) reads all 8 chunks
  constexpr int kSub = kF8 ? 2 : 4;
  for (int wid = 0; wid < kW; ++wid) {
    const int wm = wid >> 1, wn = wid & 1;
    for (int lane = 0; lane < 64; ++lane) {
      const int frow = lane & 31, fhalf = lane >> 5;
      for (int ks = 0; ks < kSub; ++ks) {
        const int nread = kF8 ? 2 : 1;
        for (int rd = 0; rd < nread; ++rd) {
          const int c = kF8 ? 4 * ks + 2 * fhalf + rd : 2 * ks + fhalf;
          for (int i = 0; i < C::kFM; ++i) {
            const int r = big_frag_row<BN, kW>(wm, i, frow);
            const int off = big_lds_off(r, c);
            CHECK(r >= 0 && r < kBigBM && off >= 0 && off + 16 <= C::kStageA, "Xq frag row %d off %d", r, off);
            if (off < 0 || off + 16 > C::kStageA) continue;
            const Tag t = lds[off / 16];
            CHECK(t.op == 0 && t.row == r && t.chunk == c, "Xq frag (%d,%d) finds (%d,%d,%d)", r, c, t.op, t.row,
                  t.chunk);
          }
          for (int j = 0; j < C::kFN; ++j) {
            const int r = big_wfrag_row<BN, kW>(wn, j, frow);
            const int off = C::kStageA + big_lds_off(r, c);
            CHECK(r >= 0 && r < BN && off >= C::kStageA && off + 16 <= C::kStage, "Wq frag row %d off %d", r, off);
            if (off < C::kStageA || off + 16 > C::kStage) continue;
            const Tag t = lds[off / 16];
            CHECK(t.op == 1 && t.row == r && t.chunk == c, "Wq frag (%d,%d) finds (%d,%d,%d)", r, c, t.op, t.row,
                  t.chunk);
          }
        }
      }
    }
  }
  // k coverage of one substep pair of lanes: chunks {2ks, 2ks+1} (int8) or
  // {4ks .. 4ks+3} (E4M3) over the two lane halves, all 8 over the stage
  int seen = 0;
  for (int ks = 0; ks < kSub; ++ks)
    for (int fhalf = 0; fhalf < 2; ++fhalf)
      for (int rd = 0; rd < (kF8 ? 2 : 1); ++rd) seen |= 1 << (kF8 ? 4 * ks + 2 * fhalf + rd : 2 * ks + fhalf);
  CHECK(seen == 0xFF, "chunks read per stage %x", seen);
  // every output column of a wave belongs to exactly one (j, rg, fhalf, e)
  std::vector<int> col(BN, 0);
  for (int wn = 0; wn < 2; ++wn)
    for (int j = 0; j < C::kFN; ++j)
      for (int rg = 0; rg < 4; ++rg)
        for (int fhalf = 0; fhalf < 2; ++fhalf)
          for (int e = 0; e < 4; ++e) {
            const int n = big_frag_col<BN, kW>(wn, j, rg, fhalf) + e;
            CHECK(n >= 0 && n < BN, "column %d", n);
            if (n >= 0 && n < BN) ++col[n];
          }
  for (int n = 0; n < BN; ++n) CHECK(col[n] == 1, "column %d held %d times", n, col[n]);
}

// The epilogue's LDS staging for output element size kEl: every staged
// element written once per band, by the lane that holds it, and copied out
// from the place it was staged, into the tile position it belongs to.
template <int BN, int kW, int kEl>
static void big_band_checks() {
  using C = BigCfg<BN, kW>;
  using B = BigBand<BN, kW, kEl>;
  g_ctx = "big band BN=" + std::to_string(BN) + " el=" + std::to_string(kEl);
  CHECK(B::kRows * B::kRowB <= C::kStage, "band %d bytes", B::kRows * B::kRowB);
  CHECK(B::kRowB % 16 == 0 && B::kColsB * B::kParts == BN, "row bytes %d", B::kRowB);
  for (int b = 0; b < C::kFM * B::kParts; ++b) {
    const int i = b / B::kParts, h = b % B::kParts;
    // staged element e of byte slot: tile row / column it holds
    std::vector<int> trow(B::kRows * B::kRowB / kEl, -1), tcol(B::kRows * B::kRowB / kEl, -1);
    for (int wid = 0; wid < kW; ++wid) {
      const int wm = wid >> 1, wn = wid & 1;
      if (!(B::kParts == 1 || wn == h)) continue;
      for (int lane = 0; lane < 64; ++lane) {
        const int frow = lane & 31, fhalf = lane >> 5;
        const int lr = wm * 32 + frow;
        for (int j = 0; j < C::kFN; ++j)
          for (int rg = 0; rg < 4; ++rg) {
            const int nl = big_frag_col<BN, kW>(wn, j, rg, fhalf);
            const int cb = (nl - h * B::kColsB) * kEl;
            CHECK(cb >= 0 && cb + 4 * kEl <= B::kRowB, "staged byte %d", cb);
            const int pc = band_chunk(cb >> 4, lr, B::kCh);
            CHECK(pc >= 0 && pc < B::kCh, "chunk %d", pc);
            const int byte = lr * B::kRowB + pc * 16 + (cb & 15);
            CHECK(byte >= 0 && byte + 4 * kEl <= B::kRows * B::kRowB && (cb & 15) + 4 * kEl <= 16, "byte %d", byte);
            if (!(byte >= 0 && byte + 4 * kEl <= B::kRows * B::kRowB)) continue;
            for (int e = 0; e < 4; ++e) {
              const int slot = byte / kEl + e;
              CHECK(trow[slot] == -1, "slot %d staged twice", slot);
              trow[slot] = big_frag_row<BN, kW>(wm, i, frow);
              tcol[slot] = nl + e;
            }
          }
      }
    }
    for (size_t s = 0; s < trow.size(); ++s) CHECK(trow[s] != -1, "staged slot %zu never written", s);
    // copy-out
    for (int c = 0; c < B::kRows * B::kCh; ++c) {
      const int lr = c / B::kCh, ch = c - lr * B::kCh;
      const int tr = band_tile_row<BN, kW>(lr, i);
      const int tc = h * B::kColsB + ch * B::kPer;
      const int byte = lr * B::kRowB + band_chunk(ch, lr, B::kCh) * 16;
      CHECK(byte >= 0 && byte + 16 <= B::kRows * B::kRowB, "copy-out byte %d", byte);
      for (int e = 0; e < B::kPer; ++e) {
        const int slot = byte / kEl + e;
        CHECK(trow[slot] == tr && tcol[slot] == tc + e, "copy-out (%d,%d) reads (%d,%d)", tr, tc + e, trow[slot],
              tcol[slot]);
      }
    }
  }
}

struct Shape {
  int64_t m, n, k;
};

// Shape checks of one prefill launch: plan p (bn, S, slice_stages, tiles),
// output element size el, y rows ldy (elements), rows16 staging or direct
// stores. `every_tile`: replay the epilogue of every tile (else of the edge
// tiles and the first, which covers every distinct masking case).
template <int BN, int kW>
static void big_shape_checks(const Shape& sh, const BigSplit& p, bool f8, int el, int64_t ldy, bool rows16,
                             bool every_tile) {
  using C = BigCfg<BN, kW>;
  const int M = (int)sh.m, N = (int)sh.n, K = (int)sh.k;
  g_ctx = "big " + std::to_string(M) + "x" + std::to_string(N) + "x" + std::to_string(K) + " BN=" +
          std::to_string(BN) + " S=" + std::to_string(p.S) + (f8 ? " e4m3" : "") + " el=" + std::to_string(el) +
          (rows16 ? " rows16" : " direct") + " ldy=" + std::to_string(ldy);
  const int nbm = (M + kBigBM - 1) / kBigBM, nbn = (N + BN - 1) / BN;
  const int total = nbm * nbn;
  const int stages = K / kBigBK;
  CHECK(K % kBigBK == 0 && K > 0, "K %d", K);
  CHECK((int64_t)total == p.tiles, "tiles %d vs plan %lld", total, (long long)p.tiles);
  // tile schedule: a bijection
  std::vector<int> seen(total, 0);
  std::vector<BigTile> tile_of(total);
  for (int t = 0; t < total; ++t) {
    const BigTile bt = big_tile(t, nbm, nbn);
    CHECK(bt.tm >= 0 && bt.tm < nbm && bt.tn >= 0 && bt.tn < nbn, "workgroup %d -> tile (%d,%d)", t, bt.tm, bt.tn);
    if (bt.tm >= 0 && bt.tm < nbm && bt.tn >= 0 && bt.tn < nbn) ++seen[bt.tm * nbn + bt.tn];
    tile_of[t] = bt;
  }
  for (int t = 0; t < total; ++t) CHECK(seen[t] == 1, "tile %d visited %d times", t, seen[t]);
  // K slices: a partition of the stages
  const bool split = p.S > 1;
  std::vector<int> stage_hits(stages, 0);
  for (int s = 0; s < p.S; ++s) {
    const BigSlice sl = big_slice(split, s, p.slice_stages, stages);
    CHECK(sl.nk >= 1 && sl.kt0 >= 0 && sl.kt0 + sl.nk <= stages, "slice %d: kt0 %d nk %d", s, sl.kt0, sl.nk);
    for (int kt = sl.kt0; kt < sl.kt0 + sl.nk && kt < stages; ++kt) ++stage_hits[kt];
  }
  for (int kt = 0; kt < stages; ++kt) CHECK(stage_hits[kt] == 1, "stage %d in %d slices", kt, stage_hits[kt]);
  // transfers: global bytes inside the operands at the first and last stage
  // of each slice (the offset is affine in the stage)
  const int64_t a_bytes = (int64_t)M * K, b_bytes = (int64_t)N * K;
  for (int t = 0; t < total; ++t) {
    const int m0 = tile_of[t].tm * kBigBM, n0 = tile_of[t].tn * BN;
    for (int s = 0; s < p.S; ++s) {
      const BigSlice sl = big_slice(split, s, p.slice_stages, stages);
      for (int kt : {sl.kt0, sl.kt0 + sl.nk - 1})
        for (int wid = 0; wid < kW; ++wid)
          for (int lane = 0; lane < 64; ++lane)
            for (int i = 0; i < C::kDma; ++i) {
              const BigDma d = big_dma<BN, kW>(i, wid, lane);
              const int64_t off = d.a ? big_dma_src(m0, d.row, M, K, kt, d.chunk)
                                      : big_dma_src(n0, d.row, N, K, kt, d.chunk);
              const int64_t lim = d.a ? a_bytes : b_bytes;
              CHECK(off >= 0 && off + 16 <= lim, "transfer at %lld of %lld (tile %d, stage %d)", (long long)off,
                    (long long)lim, t, kt);
              // the kernel's form: a buffer resource over the tile's valid
              // rows, a fixed lane offset and the stage's scalar offset
              const int tile_row0 = d.a ? m0 : n0;
              const int valid = big_tile_rows(tile_row0, d.a ? M : N, d.a ? kBigBM : BN);
              const int64_t voff = big_dma_voff(d.row, valid, K, d.chunk), soff = big_dma_soff(kt);
              const int64_t rbytes = (int64_t)valid * K;
              CHECK(valid >= 1 && rbytes < (1ll << 31), "tile resource of %lld bytes", (long long)rbytes);
              CHECK(voff >= 0 && soff >= 0 && voff + soff + 16 <= rbytes, "buffer transfer at %lld of %lld",
                    (long long)(voff + soff), (long long)rbytes);
              CHECK((int64_t)tile_row0 * K + voff + soff == off, "buffer transfer misaddressed (tile %d)", t);
              // a real row reads its own row and stage
              const int row = (d.a ? m0 : n0) + d.row;
              if (row < (d.a ? M : N))
                CHECK(off == (int64_t)row * K + (int64_t)kt * kBigBK + d.chunk * 16, "row %d misaddressed", row);
            }
    }
  }
  // split K: partial tiles and counters
  if (split) {
    CHECK(p.tiles <= kSplitMaxCounters, "%lld tiles exceed the counter region", (long long)p.tiles);
    const uint64_t pbytes64 = (uint64_t)p.S * (uint64_t)total * C::kTileBytes;
    CHECK(pbytes64 < (1ull << 31), "partial tiles %llu bytes", (unsigned long long)pbytes64);
    CHECK(big_workspace_bytes(p) == kSplitCounterBytes + pbytes64, "workspace size");
    std::vector<uint8_t> slot(pbytes64 / 16, 0);
    for (int s = 0; s < p.S; ++s)
      for (int tid_ = 0; tid_ < total; ++tid_)
        for (int wid = 0; wid < kW; ++wid)
          for (int lane = 0; lane < 64; ++lane)
            for (int q = 0; q < C::kFN * C::kFM; ++q)
              for (int rg = 0; rg < 4; ++rg) {
                const uint32_t off = big_partial_off<BN, kW>(s, total, tid_, wid, lane, q, rg);
                const uint64_t off64 = ((uint64_t)s * total + tid_) * C::kTileBytes + (uint64_t)wid * C::kWaveBytes +
                                       (uint64_t)lane * 16 + (uint64_t)(q * 4 + rg) * 1024;
                CHECK(off == off64 && off64 + 16 <= pbytes64, "partial off %u (%llu)", off,
                      (unsigned long long)off64);
                if (off64 + 16 <= pbytes64) ++slot[off64 / 16];
              }
    for (size_t i = 0; i < slot.size(); ++i)
      if (slot[i] != 1) {
        CHECK(slot[i] == 1, "partial slot %zu written %d times", i, slot[i]);
        break;
      }
  }
  // epilogue stores: inside y, every output once
  const int64_t y_elems = (int64_t)(M - 1) * ldy + N;
  const int64_t words = ((int64_t)M * N + 63) / 64;
  std::vector<uint64_t> done(every_tile ? words : 0, 0);
  auto mark = [&](int m, int n) {
    if (!every_tile) return;
    const int64_t e = (int64_t)m * N + n;
    const uint64_t bit = 1ull << (e & 63);
    CHECK(!(done[e >> 6] & bit), "output (%d,%d) stored twice", m, n);
    done[e >> 6] |= bit;
  };
  int64_t stored = 0;
  for (int t = 0; t < total; ++t) {
    const int tm = tile_of[t].tm, tn = tile_of[t].tn;
    if (!every_tile && !(t == 0 || tm == nbm - 1 || tn == nbn - 1)) continue;
    const int m0 = tm * kBigBM, n0 = tn * BN;
    // scale reads: token scales guarded by m < M; channel scales n .. n+3
    for (int tid_ = 0; tid_ < BN / 4; ++tid_) {
      const int n = n0 + 4 * tid_;
      if (n + 4 <= N) CHECK(n + 4 <= N, "w_scale");
    }
    if (rows16) {
      auto band = [&](auto band_el) {
        constexpr int kEl = decltype(band_el)::value;
        using B = BigBand<BN, kW, kEl>;
        for (int b = 0; b < C::kFM * B::kParts; ++b) {
          const int i = b / B::kParts, h = b % B::kParts;
          for (int c = 0; c < B::kRows * B::kCh; ++c) {
            const int lr = c / B::kCh, ch = c - lr * B::kCh;
            const int m = m0 + band_tile_row<BN, kW>(lr, i);
            const int n = n0 + h * B::kColsB + ch * B::kPer;
            if (m >= M || n >= N) continue;
            const int nv = n + B::kPer <= N ? B::kPer : N - n;
            const int64_t off = (int64_t)m * ldy + n;
            CHECK(off >= 0 && off + nv <= y_elems && n + nv <= N, "y store at %lld (+%d) of %lld", (long long)off, nv,
                  (long long)y_elems);
            CHECK(((off * kEl) & 15) == 0 || nv < B::kPer, "16-byte store misaligned at %lld", (long long)off);
            for (int e = 0; e < nv; ++e) mark(m, n + e);
            stored += nv;
          }
        }
      };
      if (el == 4)
        band(std::integral_constant<int, 4>());
      else
        band(std::integral_constant<int, 2>());
    } else {
      for (int wid = 0; wid < kW; ++wid) {
        const int wm = wid >> 1, wn = wid & 1;
        for (int lane = 0; lane < 64; ++lane)
          for (int j = 0; j < C::kFN; ++j)
            for (int rg = 0; rg < 4; ++rg) {
              const int n = n0 + big_frag_col<BN, kW>(wn, j, rg, lane >> 5);
              if (n >= N) continue;
              const int nvalid = std::min(4, N - n);
              for (int i = 0; i < C::kFM; ++i) {
                const int m = m0 + big_frag_row<BN, kW>(wm, i, lane & 31);
                if (m >= M) continue;
                const int64_t off = (int64_t)m * ldy + n;
                CHECK(off >= 0 && off + nvalid <= y_elems, "y store at %lld (+%d)", (long long)off, nvalid);
                for (int e = 0; e < nvalid; ++e) mark(m, n + e);
                stored += nvalid;
              }
            }
      }
    }
  }
  if (every_tile) CHECK(stored == (int64_t)M * N, "stored %lld of %lld outputs", (long long)stored, (long long)M * N);
}

// Every launch the prefill dispatch makes for this shape: int8 with the
// plan's split and unsplit (the LLM.int8() epilogue never splits), E4M3 with
// its own plan, each output element size, staged and direct stores.
static void big_shape(const Shape& sh, bool every_tile) {
  for (int f8 = 0; f8 < 2; ++f8)
    for (int split_ok = 0; split_ok < 2; ++split_ok) {
      if (f8 && !split_ok) continue;
      if (!big_suits(sh.m, sh.n, sh.k, split_ok)) continue;
      const BigSplit p = big_split(sh.m, sh.n, sh.k, f8, split_ok);
      g_ctx = "big plan";
      CHECK(p.bn == 128 || p.bn == 192 || (p.bn == 256 && !f8), "tile width %d", p.bn);
      CHECK(p.S >= 1 && p.S <= kBigMaxSplit, "S %d", p.S);
      for (int el : {2, 4})
        for (int rows16 = 0; rows16 < 2; ++rows16) {
          if (rows16 && (sh.n * el) % 16 != 0) continue;
          const int64_t ldy = rows16 ? sh.n : sh.n + 1;
          if (p.bn == 128) big_shape_checks<128, 8>(sh, p, f8, el, ldy, rows16, every_tile);
          if (p.bn == 192) big_shape_checks<192, 8>(sh, p, f8, el, ldy, rows16, every_tile);
          if (p.bn == 256) big_shape_checks<256, 8>(sh, p, f8, el, ldy, rows16, every_tile);
        }
    }
}

// ------------------------------------------------------------------- decode

// Configuration checks of the ring form (all tiles alike).
template <int kTok>
static void ring_config_checks() {
  using C = RingCfg<kTok>;
  g_ctx = "ring config tok=" + std::to_string(kTok);
  CHECK(C::kLds + 16 <= 160 * 1024, "LDS %d bytes", C::kLds + 16);
  CHECK(C::kLds >= C::kRing * C::kStage && C::kLds >= C::kRedBytes, "LDS holds the ring and the reduction");
  CHECK(C::kStage % 1024 == 0, "stage size %d", C::kStage);
  CHECK((C::kRing - 2) * C::kDma <= 63 && C::kRing >= 2, "vmcnt range");
  // one stage of transfers: every 16-byte slot once, with its tag
  std::vector<Tag> lds(C::kStage / 16);
  for (int wid = 0; wid < kDecWaves; ++wid)
    for (int lane = 0; lane < 64; ++lane)
      for (int i = 0; i < C::kDma; ++i) {
        const RingDma d = ring_dma<kTok>(i, wid, lane);
        const int off = d.dst + 16 * lane;
        CHECK(d.dst % 1024 == 0, "transfer block at %d", d.dst);
        CHECK(d.row >= 0 && d.row < (d.w ? C::kRows : kTok), "row %d", d.row);
        CHECK(d.chunk >= 0 && d.chunk < 8, "chunk %d", d.chunk);
        CHECK(off >= (d.w ? 0 : C::kStageW) && off + 16 <= (d.w ? C::kStageW : C::kStage), "lds off %d", off);
        if (off < 0 || off + 16 > C::kStage) continue;
        CHECK(off - (d.w ? 0 : C::kStageW) == big_lds_off(d.row, d.chunk), "transfer slot vs fragment layout");
        Tag& t = lds[off / 16];
        CHECK(t.op == -1, "LDS slot %d written twice", off);
        t.op = d.w ? 1 : 0;
        t.row = d.row;
        t.chunk = d.chunk;
      }
  for (size_t e = 0; e < lds.size(); ++e) CHECK(lds[e].op != -1, "LDS slot %zu never written", e);
  // fragment reads: wave q reads chunks 2q, 2q+1 of every row of its blocks
  std::vector<int> wseen((size_t)C::kRows * 8, 0), xseen((size_t)kTok * 8, 0);
  for (int q = 0; q < kDecWaves; ++q)
    for (int lane = 0; lane < 64; ++lane) {
      for (int bn = 0; bn < C::kNB; ++bn) {
        const int off = ring_frag_w<kTok>(bn, q, lane);
        CHECK(off >= 0 && off + 16 <= C::kStageW && off % 16 == 0, "w frag off %d", off);
        if (off < 0 || off + 16 > C::kStageW) continue;
        const Tag& t = lds[off / 16];
        const int row = 32 * bn + (lane & 31), chunk = 2 * q + (lane >> 5);
        CHECK(t.op == 1 && t.row == row && t.chunk == chunk, "w frag finds (%d,%d,%d)", t.op, t.row, t.chunk);
        ++wseen[(size_t)row * 8 + chunk];
      }
      for (int bm = 0; bm < C::kMB; ++bm) {
        const int off = ring_frag_x<kTok>(bm, q, lane);
        CHECK(off >= C::kStageW && off + 16 <= C::kStage && off % 16 == 0, "x frag off %d", off);
        if (off < C::kStageW || off + 16 > C::kStage) continue;
        const Tag& t = lds[off / 16];
        const int row = 32 * bm + (lane & 31), chunk = 2 * q + (lane >> 5);
        CHECK(t.op == 0 && t.row == row && t.chunk == chunk, "x frag finds (%d,%d,%d)", t.op, t.row, t.chunk);
        ++xseen[(size_t)row * 8 + chunk];
      }
    }
  for (int v : wseen) CHECK(v == 1, "w chunk read %d times", v);
  for (int v : xseen) CHECK(v == 1, "x chunk read %d times", v);
  // E4M3 fragments: wave w reads chunks 4 (w & 1) + 2 (lane / 32) + half of
  // the rows of Wq block w >> 1 (each Wq chunk once) and of every Xq block
  // (each Xq chunk twice: both Wq blocks' waves)
  std::fill(wseen.begin(), wseen.end(), 0);
  std::fill(xseen.begin(), xseen.end(), 0);
  for (int wid = 0; wid < kDecWaves; ++wid)
    for (int lane = 0; lane < 64; ++lane)
      for (int half = 0; half < 2; ++half) {
        const int chunk = 4 * (wid & 1) + 2 * (lane >> 5) + half;
        const int offw = ring_f8_frag_w<kTok>(wid, lane, half);
        CHECK(offw >= 0 && offw + 16 <= C::kStageW && offw % 16 == 0, "f8 w frag off %d", offw);
        if (offw >= 0 && offw + 16 <= C::kStageW) {
          const Tag& t = lds[offw / 16];
          const int row = 32 * (wid >> 1) + (lane & 31);
          CHECK(t.op == 1 && t.row == row && t.chunk == chunk, "f8 w frag finds (%d,%d,%d)", t.op, t.row, t.chunk);
          ++wseen[(size_t)row * 8 + chunk];
        }
        for (int bm = 0; bm < C::kMB; ++bm) {
          const int offx = ring_f8_frag_x<kTok>(bm, wid, lane, half);
          CHECK(offx >= C::kStageW && offx + 16 <= C::kStage && offx % 16 == 0, "f8 x frag off %d", offx);
          if (offx < C::kStageW || offx + 16 > C::kStage) continue;
          const Tag& t = lds[offx / 16];
          const int row = 32 * bm + (lane & 31);
          CHECK(t.op == 0 && t.row == row && t.chunk == chunk, "f8 x frag finds (%d,%d,%d)", t.op, t.row, t.chunk);
          ++xseen[(size_t)row * 8 + chunk];
        }
      }
  for (int v : wseen) CHECK(v == 1, "f8 w chunk read %d times", v);
  for (int v : xseen) CHECK(v == 2, "f8 x chunk read %d times", v);
  // E4M3 reduction slots: what each holds; outputs read from waves 2 bn, 2 bn + 1
  std::vector<int> holds8((size_t)kDecWaves * C::kSlotsF8, -1);
  for (int wid = 0; wid < kDecWaves; ++wid)
    for (int bm = 0; bm < C::kMB; ++bm)
      for (int rg = 0; rg < 4; ++rg)
        for (int lane = 0; lane < 64; ++lane) {
          const int slot = ring_f8_slot<kTok>(bm, rg, lane);
          CHECK(slot >= 0 && slot < C::kSlotsF8, "f8 slot %d", slot);
          if (slot < 0 || slot >= C::kSlotsF8) continue;
          int& h = holds8[(size_t)wid * C::kSlotsF8 + slot];
          CHECK(h == -1, "f8 slot written twice");
          h = (32 * bm + (lane & 31)) * 64 + 32 * (wid >> 1) + 8 * rg + 4 * (lane >> 5);
        }
  CHECK(C::kLds >= kDecWaves * C::kSlotsF8 * 16, "f8 reduction fits");
  for (int tid = 0; tid < 256; ++tid)
    for (int g = 0; g < C::kNG; ++g) {
      const int ml = ring_tok<kTok>(tid), nl = ring_col<kTok>(tid, g);
      const int slot = ring_f8_read_slot<kTok>(ml, nl);
      const int w0 = 2 * (nl >> 5);
      CHECK(slot >= 0 && slot < C::kSlotsF8 && w0 + 1 < kDecWaves, "f8 read slot %d", slot);
      if (slot < 0 || slot >= C::kSlotsF8 || w0 + 1 >= kDecWaves) continue;
      for (int w = w0; w < w0 + 2; ++w)
        CHECK(holds8[(size_t)w * C::kSlotsF8 + slot] == ml * 64 + nl, "f8 read slot content");
    }
  // reduction slots: what each holds, and where the epilogue reads
  std::vector<int> holds(C::kSlots, -1);  // token * 64 + first output
  for (int bn = 0; bn < C::kNB; ++bn)
    for (int bm = 0; bm < C::kMB; ++bm)
      for (int rg = 0; rg < 4; ++rg)
        for (int lane = 0; lane < 64; ++lane) {
          const int slot = ring_slot<kTok>(bn, bm, rg, lane);
          CHECK(slot >= 0 && slot < C::kSlots, "slot %d", slot);
          if (slot < 0 || slot >= C::kSlots) continue;
          CHECK(holds[slot] == -1, "slot %d written twice", slot);
          holds[slot] = (32 * bm + (lane & 31)) * 64 + 32 * bn + 8 * rg + 4 * (lane >> 5);
        }
  std::vector<int> outs((size_t)kTok * 64, 0);
  for (int tid = 0; tid < 256; ++tid)
    for (int g = 0; g < C::kNG; ++g) {
      const int ml = ring_tok<kTok>(tid), nl = ring_col<kTok>(tid, g);
      CHECK(ml >= 0 && ml < kTok && nl >= 0 && nl + 4 <= 64 && nl % 4 == 0, "epilogue (%d,%d)", ml, nl);
      if (ml < 0 || ml >= kTok || nl < 0 || nl + 4 > 64) continue;
      const int slot = ring_read_slot<kTok>(ml, nl);
      CHECK(slot >= 0 && slot < C::kSlots && holds[slot] == ml * 64 + nl, "read slot %d", slot);
      if (g > 0) CHECK(nl == ring_col<kTok>(tid, g - 1) + 4, "a thread's outputs are consecutive");
      for (int e = 0; e < 4; ++e) ++outs[(size_t)ml * 64 + nl + e];
    }
  for (int v : outs) CHECK(v == 1, "tile output covered %d times", v);
}

// One shape of the ring form.
template <int kTok>
static void ring_shape(int M, int N, int K, const DecodePlan& p) {
  using C = RingCfg<kTok>;
  CHECK(p.tb == 1 || kTok == 64, "token layers with %d-token tiles", kTok);
  CHECK(dec_ring_tok(M) == kTok, "token tile");
  const int steps = K / kDecStep;
  // transfers over each slice, inside the operands
  for (int s = 0; s < p.S; ++s) {
    const DecSlice sl = dec_slice(s, p.slice_steps, K);
    CHECK(sl.nsl >= 1 && sl.step0 + sl.nsl <= steps, "slice %d", s);
    for (int wid = 0; wid < kDecWaves; ++wid)
      for (int lane = 0; lane < 64; ++lane)
        for (int i = 0; i < C::kDma; ++i) {
          const RingDma d = ring_dma<kTok>(i, wid, lane);
          for (int tile = 0; tile < p.tiles; tile += (p.tiles > 2 ? p.tiles - 1 : 1))
            for (int z = 0; z < p.tb; ++z) {
              const int64_t base = d.w ? big_dma_src(tile * C::kRows, d.row, N, K, sl.step0, d.chunk)
                                       : big_dma_src(z * 64, d.row, M, K, sl.step0, d.chunk);
              const int64_t last = base + (int64_t)(sl.nsl - 1) * kDecStep;
              const int64_t size = (int64_t)(d.w ? N : M) * K;
              CHECK(base >= 0 && last + 16 <= size, "transfer outside the operand");
            }
        }
  }
  // partial tiles and outputs
  const bool split = p.S > 1;
  const int nctr = p.tiles * p.tb;
  const uint64_t pbytes = (uint64_t)p.S * nctr * C::kTileBytes;
  if (split) {
    CHECK(nctr <= kSplitMaxCounters, "counters %d", nctr);
    CHECK(pbytes < (1ull << 31), "partials %llu bytes", (unsigned long long)pbytes);
    CHECK(dec_workspace_bytes(p, M, N, true) == kSplitCounterBytes + pbytes, "workspace size");
  }
  std::vector<uint8_t> pw(split ? pbytes / 16 : 0, 0);
  std::vector<uint8_t> out((size_t)M * N, 0);
  for (int z = 0; z < p.tb; ++z)
    for (int tile = 0; tile < p.tiles; ++tile) {
      const int ctr = z * p.tiles + tile;
      for (int tid = 0; tid < 256; ++tid)
        for (int g = 0; g < C::kNG; ++g) {
          if (split)
            for (int s = 0; s < p.S; ++s) {
              const uint32_t off = ring_partial_off(s, nctr, ctr, g, tid, C::kTileBytes);
              CHECK(off % 16 == 0 && off + 16 <= pbytes, "partial off %u", off);
              if (off + 16 <= pbytes) ++pw[off / 16];
            }
          const int m = z * 64 + ring_tok<kTok>(tid), n = tile * C::kRows + ring_col<kTok>(tid, g);
          if (m >= M || n >= N) continue;
          for (int e = 0; e < std::min(4, N - n); ++e) ++out[(size_t)m * N + n + e];
        }
    }
  for (size_t e = 0; e < out.size(); ++e)
    if (out[e] != 1) {
      CHECK(out[e] == 1, "output %zu stored %d times", e, out[e]);
      break;
    }
  for (size_t e = 0; e < pw.size(); ++e)
    if (pw[e] != 1) {
      CHECK(pw[e] == 1, "partial slot %zu written %d times", e, pw[e]);
      break;
    }
}

static void decode_shape(const Shape& sh, bool f8) {
  const int M = (int)sh.m, N = (int)sh.n, K = (int)sh.k;
  g_ctx = "decode " + std::to_string(M) + "x" + std::to_string(N) + "x" + std::to_string(K) + (f8 ? " e4m3" : "");
  if (!decode_suits(sh.m, sh.n, sh.k, f8)) return;
  const DecodePlan p = decode_plan(sh.m, sh.n, sh.k);
  if (dec_ring(sh.m, f8)) {
    CHECK(p.S >= 1 && p.tiles == (N + kDecRows - 1) / kDecRows && p.tb == (M + 63) / 64, "plan");
    if (dec_ring_tok(sh.m) == 32)
      ring_shape<32>(M, N, K, p);
    else
      ring_shape<64>(M, N, K, p);
    return;
  }
  const int kMB = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  const int kTok = 16 * kMB;
  const int steps = K / kDecStep;
  CHECK(p.ns >= 1 && p.ns <= kDecMaxNS, "steps per wave %d outside the template range", p.ns);
  CHECK(p.S >= 1 && p.tiles == (N + kDecRows - 1) / kDecRows && p.tb == (M + 63) / 64, "plan");
  CHECK(p.tb == 1 || kMB == 4, "token blocks %d with %d-token fragments", p.tb, kTok);
  const int kb_max = dec_kb(f8, 63), kh = dec_khalf(f8);
  CHECK(kb_max + kh + 16 <= kDecStep && dec_kb(f8, 0) == 0, "lane k bytes");
  // steps: every slice step loaded by exactly one (wave, i) whose product counts
  std::vector<int> hit(steps, 0);
  for (int s = 0; s < p.S; ++s) {
    const DecSlice sl = dec_slice(s, p.slice_steps, K);
    CHECK(sl.nsl >= 1 && sl.step0 + sl.nsl <= steps, "slice %d: %d + %d", s, sl.step0, sl.nsl);
    CHECK(sl.nsl <= kDecWaves * p.ns, "slice of %d steps over %d waves x %d", sl.nsl, kDecWaves, p.ns);
    for (int wid = 0; wid < kDecWaves; ++wid)
      for (int i = 0; i < p.ns; ++i) {
        const int st = dec_step(wid, i, sl.nsl);
        CHECK(st >= 0 && st < sl.nsl, "step %d", st);
        const int64_t off = (int64_t)(sl.step0 + st) * kDecStep;
        CHECK(off + kb_max + kh + 16 <= K, "load past the row end");
        if (dec_step_valid(wid, i, sl.nsl)) {
          CHECK(st == wid + kDecWaves * i, "valid step clamped");
          if (sl.step0 + st < steps) ++hit[sl.step0 + st];
        }
      }
  }
  for (int st = 0; st < steps; ++st) CHECK(hit[st] == 1, "step %d counted %d times", st, hit[st]);
  // operand rows
  for (int tile = 0; tile < p.tiles; ++tile)
    for (int lane = 0; lane < 64; ++lane)
      for (int g = 0; g < 4; ++g) {
        const int r = dec_w_row(tile * kDecRows, g, lane, N);
        CHECK(r >= 0 && r < N, "Wq row %d", r);
      }
  for (int z = 0; z < p.tb; ++z)
    for (int lane = 0; lane < 64; ++lane)
      for (int mb = 0; mb < kMB; ++mb) {
        const int r = dec_x_row(z * 64, mb, lane, M);
        CHECK(r >= 0 && r < M, "Xq row %d", r);
        if (z * 64 + 16 * mb + (lane & 15) < M) CHECK(r == z * 64 + 16 * mb + (lane & 15), "Xq row clamped");
      }
  // LDS reduction: red[wave][tok][4 quad + e], each quad read where written
  {
    std::vector<int> tag((size_t)kDecWaves * kTok * 16, -1);
    for (int wid = 0; wid < kDecWaves; ++wid)
      for (int g = 0; g < 4; ++g)
        for (int mb = 0; mb < kMB; ++mb)
          for (int lane = 0; lane < 64; ++lane) {
            const int tok = 16 * mb + (lane & 15);
            const int quad = dec_red_quad(g, lane, tok);
            CHECK(tok < kTok && quad >= 0 && quad < 16, "red (%d,%d)", tok, quad);
            const size_t at = ((size_t)wid * kTok + tok) * 16 + quad;
            CHECK(tag[at] == -1, "red quad written twice");
            tag[at] = 4 * g + (lane >> 4);  // the rows 4 x this .. +3 of the tile
          }
    for (int tid = 0; tid < 256; ++tid)
      for (int j = 0; j < kMB; ++j) {
        const int q = tid & 15, tok = (tid >> 4) + 16 * j;
        const int sq = q ^ (tok & 15);
        for (int w = 0; w < kDecWaves; ++w) CHECK(tag[((size_t)w * kTok + tok) * 16 + sq] == q, "red read");
      }
  }
  // outputs and partial tiles
  const int64_t ldy = N;
  std::vector<uint8_t> out((size_t)M * N, 0);
  const bool split = p.S > 1;
  const uint64_t pbytes = (uint64_t)p.S * M * N * 4;
  if (split) {
    CHECK((int64_t)p.tiles * p.tb <= kSplitMaxCounters, "counters %d", p.tiles * p.tb);
    CHECK(pbytes < (1ull << 31), "partials %llu bytes", (unsigned long long)pbytes);
    CHECK(dec_workspace_bytes(p, M, N) == kSplitCounterBytes + pbytes, "workspace size");
  }
  std::vector<uint8_t> pw(split ? pbytes / 4 : 0, 0);
  for (int z = 0; z < p.tb; ++z)
    for (int tile = 0; tile < p.tiles; ++tile) {
      const int ctr = z * p.tiles + tile;
      if (split) CHECK(ctr >= 0 && ctr < p.tiles * p.tb, "counter %d", ctr);
      for (int tid = 0; tid < 256; ++tid) {
        const int n = tile * kDecRows + 4 * (tid & 15);
        for (int j = 0; j < kMB; ++j) {
          const int m = z * 64 + (tid >> 4) + 16 * j;
          if (m >= M || n >= N) continue;
          const int nv = std::min(4, N - n);
          CHECK((int64_t)m * ldy + n + nv <= (int64_t)M * ldy, "y store");
          for (int e = 0; e < nv; ++e) ++out[(size_t)m * N + n + e];
          if (!split) continue;
          for (int s = 0; s < p.S; ++s) {
            const uint32_t off = dec_partial_off(s, M, N, m, n);
            const uint64_t off64 = (((uint64_t)s * M + m) * N + n) * 4;
            CHECK(off == off64 && off64 + 4 * nv <= pbytes, "partial off");
            for (int e = 0; e < nv; ++e) ++pw[off64 / 4 + e];
          }
          // the reducer's eight-slice rounds: slices past S read beyond the
          // buffer (zero) and never wrap into it
          const uint32_t off0 = dec_partial_off(0, M, N, m, n);
          const uint32_t sstride = dec_partial_off(1, M, N, 0, 0);
          for (int s = 0; s < p.S; s += 8)
            for (int u = 0; u < 8; ++u) {
              const uint64_t o64 = (uint64_t)off0 + (uint64_t)(s + u) * sstride;
              CHECK(o64 < (1ull << 32), "reducer offset wraps");
              if (s + u >= p.S) CHECK(o64 >= pbytes, "read past the last slice lands in the buffer");
            }
        }
      }
    }
  for (size_t e = 0; e < out.size(); ++e)
    if (out[e] != 1) {
      CHECK(out[e] == 1, "output %zu stored %d times", e, out[e]);
      break;
    }
  for (size_t e = 0; e < pw.size(); ++e)
    if (pw[e] != 1) {
      CHECK(pw[e] == 1, "partial word %zu written %d times", e, pw[e]);
      break;
    }
}

int main() {
  big_config_checks<128, 8, false>();
  big_config_checks<192, 8, false>();
  big_config_checks<256, 8, false>();
  big_config_checks<128, 8, true>();
  big_config_checks<192, 8, true>();
  big_config_checks<256, 4, true>();  // E4M3 256-column tiles on four waves
  big_band_checks<128, 8, 2>();
  big_band_checks<128, 8, 4>();
  big_band_checks<192, 8, 2>();
  big_band_checks<192, 8, 4>();
  big_band_checks<256, 8, 2>();
  big_band_checks<256, 4, 2>();
  big_band_checks<256, 4, 4>();
  big_band_checks<256, 8, 4>();
  ring_config_checks<32>();
  ring_config_checks<64>();

  // the workloads' prefill GEMMs (QKV, gate/up, down, LLM.int8()), replayed
  // at the edge tiles; ragged and split shapes replayed tile by tile
  const Shape workloads[] = {{2048, 6144, 4096}, {8192, 28672, 4096}, {8192, 4096, 14336}, {4096, 8192, 8192}};
  for (const Shape& s : workloads) big_shape(s, false);
  const Shape ragged[] = {
      {256, 4096, 128},   {257, 4100, 256},   {300, 4104, 1152},  {511, 6144, 4096},  {1000, 200, 512},
      {1024, 6144, 4096}, {512, 14336, 4096}, {1024, 4096, 14336}, {136, 28672, 4096}, {192, 4096, 14336},
      {176, 6144, 4096},  {256, 4096, 14336}, {640, 1640, 2560},  {2048, 196, 384},   {777, 1000, 1280},
      {129, 14336, 4096}, {4096, 192, 128},
  };
  for (const Shape& s : ragged) big_shape(s, true);

  // decode: the workloads' token counts on both MLP projections, and ragged
  const int toks[] = {1, 2, 8, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 96, 100, 128, 192, 255, 256};
  const Shape layers[] = {{0, 14336, 4096}, {0, 4096, 14336}, {0, 6144, 4096}, {0, 512, 256},   {0, 28672, 4096},
                          {0, 100, 128},    {0, 4100, 1152},  {0, 64, 128},    {0, 1, 128},     {0, 8192, 8192},
                          {0, 28672, 8192}, {0, 16448, 8192}, {0, 14336, 14336}, {0, 8256, 4160}};
  for (int m : toks)
    for (const Shape& l : layers)
      for (int f8 = 0; f8 < 2; ++f8) decode_shape(Shape{m, l.n, l.k}, f8);

  if (g_fail) {
    fprintf(stderr, "%d of %lld checks failed\n", g_fail, g_checks);
    return 1;
  }
  printf("OK %lld\n", g_checks);
  return 0;
}
