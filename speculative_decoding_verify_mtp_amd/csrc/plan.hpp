// Host-side launch planning of the verify attention: argument checks, the
// choice of partial kernel and its split plan, and the workspace layout.
// Included by mtp_verify.hip only (functions in an anonymous namespace).
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "attn_stream.hpp"
#include "attn_valu.hpp"
#include "common.hpp"
#include "mtp_verify.h"

namespace {

using namespace mtpv;

// Committed tokens per split when the caller does not fix it: enough work
// items to fill 256 CUs several times over (1024 workgroups of the LDS kernel,
// 2048 single-wave items otherwise), no longer than 2048 tokens, and at least
// twice the rows of an item (the partial a split writes, rows x (D+2) x 4
// bytes, then stays below half of the K/V it reads, split x 4D bytes).
constexpr long kTargetWorkgroups = 1024;
constexpr long kTargetWaves = 2048;
constexpr int kMinSplit = 32;  // one 32-key stage: short contexts are latency-bound
constexpr int kMaxSplit = 2048;

enum Kernel { kValu = 0, kMfmaDirect = 1, kMfmaLds = 2, kMfmaStream = 3, kMfmaNested = 4, kMfmaNestedStream = 5 };

// Kernels that write the stream layout (pieces per range and segment, a segment table).
inline bool stream_layout(int kernel) { return kernel == kMfmaStream || kernel == kMfmaNestedStream; }

// Stream kernel: persistent grid of two workgroups per compute unit of
// gfx950's 256, rounded down to a multiple of Hkv, each workgroup streaming
// at least kMinStreamStages stages.  Two per CU with every CU equally loaded
// is what the ragged batch measured fastest (512 workgroups 908 us; 768,
// three per CU, 968 us: more page streams open at once; 576 or 640, some CUs
// holding a third workgroup of equal length, 1131 and 1054 us; 384, 1022 us).
constexpr int kCUs = 256;
constexpr int kStreamWgsPerCU = 2;
constexpr long kMinStreamStages = 2;
// Length of a first-dispatch-round range relative to the others (two
// workgroups per CU; ragged batch: equal ranges 900 us, first-round share of
// the list 0.53 / 0.55 / 0.57 / 0.59: 882 / 872 / 878 / 908 us).
constexpr int kFirstRoundNum = 5, kFirstRoundDen = 4;
// Fewer than kStreamMinB sequences take the stream kernel when its ranges
// would hold at least this many stages.
constexpr long kMinRangeStages = 4;
// Stream-layout combine: segments of at most this many pieces (estimated)
// are folded four rows per wave, longer ones one row per wave.
constexpr long kGroupedMaxPieces = 12;
// Batches of at least this many sequences take the stream kernel; fewer
// do when its ranges are long enough (kMinRangeStages).
constexpr int kStreamMinB = 8;

struct Plan {
  Kernel kernel;   // VALU (fp32, or < 16 rows), MFMA with direct loads (D=64), MFMA + LDS ring (D=128)
  bool mfma;       // bf16 with >= 16 rows per KV head
  int g, R;        // group size, rows per KV head (W * g)
  int RB;          // MFMA row tiles per wave (1, 2 or 4; the per-split LDS kernel runs 1)
  int NR;          // row-tile groups (waves) per workgroup (LDS kernel; 1 wave per item otherwise)
  int KS;          // key slices per workgroup (LDS kernel: NR * KS waves)
  int nRB;         // row blocks (MFMA) or row chunks (VALU) per KV head
  int S;           // committed tokens per split (past the first n1 splits)
  int n1, S1;      // the first n1 splits hold S1 tokens each
  int max_splits;  // splits of the longest context
  int G;           // stream kernel: workgroups
  int h1;          // stream kernel: ranges per head in the first dispatch round (0: equal ranges)
  bool piece_rows; // stream layout with many pieces per segment: the combine takes a row per wave
  int nts, nseg, rows_block;
  size_t acc_bytes, ml_offset, ml_bytes, seg_offset, seg_bytes;
  size_t tgt_offset, tgt_bytes;  // the step's row targets (B * W int32)
  size_t ws_bytes;               // the whole workspace
};

mtp_status check_shape(const mtp_shape* s) {
  if (s == nullptr) return MTP_ERR_NULL;
  if (s->B < 0 || s->B > 65535) return MTP_ERR_SHAPE;
  if (s->W < 1 || s->W > MTP_MAX_W) return MTP_ERR_SHAPE;
  if (s->Hkv < 1 || s->Hq < 1 || s->Hq % s->Hkv != 0) return MTP_ERR_SHAPE;
  if (s->num_pages < 0 || s->max_pages_per_seq < 0 || s->max_ctx_len < 0) return MTP_ERR_SHAPE;
  if ((int64_t)s->max_ctx_len > (int64_t)s->max_pages_per_seq * MTP_PAGE_SIZE) return MTP_ERR_SHAPE;
  if (s->max_ctx_len > 0 && s->num_pages < 1) return MTP_ERR_SHAPE;  // committed keys need pages
  if (s->seg_lookback < -1) return MTP_ERR_SHAPE;
  if (s->split_tokens < 0 || s->split_tokens % 32 != 0 || s->split_tokens > kMaxSplit)
    return MTP_ERR_SHAPE;
  if (!(s->scale >= 0.f) || isinf(s->scale)) return MTP_ERR_SHAPE;
  if (s->page_size != MTP_PAGE_SIZE) return MTP_ERR_UNSUPPORTED;
  if (s->D != 64 && s->D != 128) return MTP_ERR_UNSUPPORTED;
  if (s->dtype != MTP_F32 && s->dtype != MTP_BF16) return MTP_ERR_UNSUPPORTED;
  return MTP_OK;
}

int pow2_ceil(long x) {
  int p = 1;
  while (p < x && p < (1 << 30)) p <<= 1;
  return p;
}

// `nested`: the plan of the nested-cache kernel (bf16, D = 128, LDS ring):
// workgroups shaped as for the bf16 LDS kernel (fewer rows than a tile are
// padded to one).
Plan make_plan(const mtp_shape& s, bool nested = false) {
  Plan pl;
  pl.g = s.Hq / s.Hkv;
  pl.R = s.W * pl.g;
  pl.mfma = nested || (s.dtype == MTP_BF16 && pl.R >= 16);
  pl.NR = 1;
  pl.KS = 1;
  const int tiles = (pl.R + 15) / 16;
  if (nested) {
    pl.kernel = kMfmaNested;
    pl.NR = tiles >= 3 ? 4 : tiles;
    const int per = (tiles + pl.NR - 1) / pl.NR;
    pl.RB = per >= 2 ? 2 : 1;
    pl.nRB = (tiles + pl.NR * pl.RB - 1) / (pl.NR * pl.RB);
  } else if (pl.mfma && s.D == 128) {
    // One workgroup of NR waves shares each K/V stage; wave w owns RB row
    // tiles.  Up to 4 waves x 2 tiles = 128 rows per row block.
    pl.kernel = kMfmaLds;
    pl.NR = tiles >= 3 ? 4 : tiles;
    const int per = (tiles + pl.NR - 1) / pl.NR;
    pl.RB = per >= 2 ? 2 : 1;
    pl.nRB = (tiles + pl.NR * pl.RB - 1) / (pl.NR * pl.RB);
  } else if (pl.mfma) {
    // Row tiles per wave: 1, 2 or 4 (a third tile is padded to four so the
    // K/V stream is still read once).
    pl.kernel = kMfmaDirect;
    pl.RB = tiles >= 3 ? 4 : tiles;
    pl.nRB = (tiles + pl.RB - 1) / pl.RB;
  } else {
    pl.kernel = kValu;
    pl.RB = 0;
    pl.nRB = (pl.R + kValuRows - 1) / kValuRows;
  }
  if (s.split_tokens > 0) {
    pl.S = s.split_tokens;
  } else {
    const bool wg = pl.kernel == kMfmaLds || pl.kernel == kMfmaNested;
    const long target = wg ? kTargetWorkgroups : kTargetWaves;
    const int rows_item = wg ? 16 * pl.NR * pl.RB : pl.kernel == kMfmaDirect ? 16 * pl.RB : kValuRows;
    const long work = (long)s.B * s.Hkv * pl.nRB * (long)(s.max_ctx_len > 0 ? s.max_ctx_len : 1);
    int S = pow2_ceil((work + target - 1) / target);
    const int floor_rows = pow2_ceil(2L * rows_item);
    S = S < floor_rows ? floor_rows : S;
    pl.S = S < kMinSplit ? kMinSplit : (S > kMaxSplit ? kMaxSplit : S);
  }
  pl.nts = (s.W + 31) / 32;
  bool stream_shape = (pl.kernel == kMfmaLds || pl.kernel == kMfmaNested) && s.B >= kStreamMinB &&
                      s.B <= kStreamMaxB;
  // Fewer sequences with one row tile per wave: the stream schedule still
  // pays once each of its ranges holds a few stages (whole steps: one
  // sequence of 32000 tokens 52.0 -> 42.9 us, two of 8000 33.9 -> 29.0 us,
  // four of 16000 77.1 -> 74.2 us; one of 4096 with 32 rows per head, about
  // two stages per range, 14.4 -> 18.6 us, so it stays per split).  The
  // nested kernels alike (attention: 49.1 -> 41.3 us, 32.9 -> 29.2 us).
  if ((pl.kernel == kMfmaLds || pl.kernel == kMfmaNested) && s.B >= 1 && s.B < kStreamMinB &&
      pl.RB == 1 && s.split_tokens == 0) {
    const long seg_stages = (long)(s.max_ctx_len + 31) / 32 + pl.nts;
    const long upper_h = (long)s.B * pl.nRB * seg_stages;
    const long slots_h = std::max(1L, (long)kCUs * kStreamWgsPerCU / s.Hkv);
    const long Gh = std::max(1L, std::min((upper_h + kMinStreamStages - 1) / kMinStreamStages, slots_h));
    stream_shape = upper_h >= kMinRangeStages * Gh;
  }
  // Per-split LDS kernel with one or two row tiles per workgroup: two key
  // slices (each wave reduces half of the stages) when every stage of a split
  // fits the ring.  The automatic split then also grows, within the ring, until
  // a row has at most kCombineFast splits (the combine's first batch), which
  // halves the partial writes and drops a combine round trip.
  const int ks_cap = 32 * (kLdsStages - pl.nts);  // longest split whose stages all fit the ring
  if (pl.kernel == kMfmaLds && !stream_shape && pl.RB == 1 && pl.NR <= 2) {
    if (s.split_tokens == 0 && pl.S < ks_cap) {
      const long want = ((long)(s.max_ctx_len + kCombineFast - 1) / kCombineFast + 31) / 32 * 32;
      pl.S = (int)std::max<long>(pl.S, std::min<long>(ks_cap, want));
    }
    if (pl.S <= ks_cap) pl.KS = 2;
  }
  pl.n1 = 0;
  pl.S1 = pl.S;
  pl.max_splits = num_splits(s.max_ctx_len, pl.S, 0, pl.S);
  pl.G = 0;
  pl.h1 = 0;
  pl.piece_rows = false;
  pl.nseg = s.Hkv * pl.nRB;
  pl.rows_block = 16 * pl.NR * pl.RB;
  size_t rows = (size_t)s.B * pl.max_splits * s.Hkv * pl.R;
  if (stream_shape) {
    // The nested stream kernel runs one row tile per wave: row blocks of at
    // most 64 rows, a segment each.
    const bool nested_rb1 = pl.kernel == kMfmaNested && pl.RB == 2;
    const int nrb = nested_rb1 ? (tiles + pl.NR - 1) / pl.NR : pl.nRB;
    // stage count bound from max_ctx_len; the device splits the true count
    const long seg_stages = (long)(s.max_ctx_len + 31) / 32 + pl.nts;
    const long upper = (long)s.B * s.Hkv * nrb * seg_stages;
    if (upper < (1L << 30) && s.Hkv <= 65535) {
      if (pl.kernel == kMfmaNested) {
        pl.kernel = kMfmaNestedStream;
        if (nested_rb1) {
          pl.RB = 1;
          pl.nRB = nrb;
          pl.nseg = s.Hkv * pl.nRB;
          pl.rows_block = 16 * pl.NR;
        }
      } else {
        pl.kernel = kMfmaStream;
      }
      // G = Hkv * Gh: each KV head's list is cut into Gh ranges
      // (two row tiles per wave take a SIMD's registers: one workgroup per CU)
      const long slots = (long)kCUs * (pl.RB == 1 ? kStreamWgsPerCU : 1);
      const long per = s.split_tokens > 0 ? s.split_tokens / 32 : kMinStreamStages;
      const long upper_h = upper / s.Hkv;
      long Gh = (upper_h + per - 1) / per;
      const long slots_h = slots / s.Hkv > 0 ? slots / s.Hkv : 1;
      if (s.split_tokens == 0 && Gh > slots_h) Gh = slots_h;
      const long max_h = 65535 / s.Hkv;
      pl.G = (int)((Gh < 1 ? 1 : (Gh > max_h ? max_h : Gh)) * s.Hkv);
      // Two workgroups per CU: the G - 256 workgroups past the first round
      // share CUs with first-round ones, whose ranges are made longer.
      if (s.split_tokens == 0 && pl.RB == 1 && pl.G > kCUs) pl.h1 = kCUs / s.Hkv;
      // pieces per segment: about one per range the segment crosses
      const long per_seg = (pl.G / s.Hkv + (long)s.B * pl.nRB - 1) / ((long)s.B * pl.nRB) + 1;
      pl.piece_rows = per_seg > kGroupedMaxPieces;
      rows = ((size_t)pl.G + (size_t)s.B * pl.nseg) * pl.rows_block;
    }
  }
  // Per-split LDS kernel with two row tiles per wave (more than 64 rows per
  // KV head): the split stays sized for 128-row workgroups, but each is run
  // as two workgroups of one row tile per wave.  Two row tiles per wave need
  // all 512 registers of a SIMD lane, so a compute unit holds one such
  // workgroup (one wave per SIMD, nothing to overlap a wave's stage chain
  // with); one tile per wave leaves room for two workgroups per CU.  The two
  // row blocks of a (split, head) read the same K/V; the kernel places them
  // eight workgroups apart, on the same XCD, so the second read is served
  // by that XCD's L2 (llama3_8b_tree partial 23.2 -> 20.6 us).
  if ((pl.kernel == kMfmaLds || pl.kernel == kMfmaNested) && pl.RB == 2) {
    pl.RB = 1;
    pl.nRB = (tiles + pl.NR - 1) / pl.NR;
  }
  // One sequence whose items fill two workgroups per CU: the dispatcher
  // places items 0 .. 255 one per CU first, and a SIMD issues the older of
  // two ready waves first, so the second item of each CU ends last (per
  // workgroup clocks on llama3_8b_tree: first-stage data 5.0 vs 9.0 us after
  // the launch, ends 15.7 vs 19.4 us).  The splits of the first round
  // (splits < n1: items are ordered by split) then hold S + d tokens and the
  // rest S - d, d ~ S / 9 (a length ratio near 5 / 4).
  if (s.split_tokens == 0 && s.B == 1 && pl.kernel == kMfmaLds && pl.KS == 1 && pl.RB == 1) {
    const long items = (long)pl.max_splits * s.Hkv * pl.nRB;
    const int n1 = (int)(kCUs / ((long)s.Hkv * pl.nRB));
    const int d = 32 * (int)lround(pl.S / (9.0 * 32));
    if (items > kCUs && items <= 2L * kCUs && n1 >= 1 && d > 0 && pl.S + d <= kMaxSplit) {
      pl.n1 = n1;
      pl.S1 = pl.S + d;
      pl.S -= d;
      pl.max_splits = num_splits(s.max_ctx_len, pl.S, pl.n1, pl.S1);
      rows = (size_t)s.B * pl.max_splits * s.Hkv * pl.R;
    }
  }
  pl.acc_bytes = rows * s.D * sizeof(float);
  pl.ml_offset = (pl.acc_bytes + 255) & ~(size_t)255;
  pl.ml_bytes = rows * 2 * sizeof(float);
  pl.seg_offset = (pl.ml_offset + pl.ml_bytes + 255) & ~(size_t)255;
  pl.seg_bytes = stream_layout(pl.kernel) ? (size_t)s.B * pl.nseg * 2 * sizeof(int) : 0;
  pl.tgt_offset = (pl.seg_offset + pl.seg_bytes + 255) & ~(size_t)255;
  pl.tgt_bytes = (size_t)s.B * s.W * sizeof(int32_t);
  pl.ws_bytes = pl.tgt_offset + pl.tgt_bytes;
  return pl;
}

// The step's target prologue (AttnParams::logits): on the per-split LDS
// kernel, whose first B * W workgroups find one logits row's argmax each,
// for rows the acceptance would reduce from registers (V <= kRegV, V % 4 ==
// 0, 16-byte aligned).
bool step_target_prologue(const Plan& pl, const mtp_shape& s, const float* logits, int V) {
  const long wgs = (long)pl.max_splits * s.Hkv * pl.nRB * s.B;
  return pl.kernel == kMfmaLds && logits != nullptr && V >= 1 && V <= kRegV && V % 4 == 0 &&
         ((uintptr_t)logits & 15) == 0 && (long)s.B * s.W <= wgs;
}

}  // namespace
