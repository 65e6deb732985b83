// Host side of libmtpverify: argument validation, split-K planning and
// kernel launches for the C ABI declared in include/mtp_verify.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <math.h>
#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "accept_commit.hpp"
#include "attn_lds.hpp"
#include "attn_mfma.hpp"
#include "attn_stream.hpp"
#include "attn_valu.hpp"
#include "combine.hpp"
#include "common.hpp"
#include "host_checks.hpp"
#include "hybrid.hpp"
#include "nested.hpp"
#include "tree.hpp"
#include "plan.hpp"
#include "attn_nested_lds.hpp"
#include "attn_nested_stream.hpp"
#include "mtp_verify.h"

namespace {

using namespace mtpv;

mtp_status launch_status() {
  return hipGetLastError() == hipSuccess ? MTP_OK : MTP_ERR_HIP;
}

}  // namespace

extern "C" {

int32_t mtp_abi_version(void) { return MTP_ABI_VERSION; }

const char* mtp_status_string(int32_t status) {
  switch (status) {
    case MTP_OK: return "ok";
    case MTP_ERR_NULL: return "a required pointer is NULL";
    case MTP_ERR_SHAPE: return "a size is out of range or inconsistent";
    case MTP_ERR_UNSUPPORTED: return "unsupported head dim, dtype or page size";
    case MTP_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MTP_ERR_HIP: return "HIP runtime error at launch";
    case MTP_ERR_CONFLICT: return "a commit slot is mapped twice or is another sequence's";
    case MTP_ERR_SCRATCH: return "the shape needs more than the library's fixed 64 MiB device scratch";
    default: return "unknown status";
  }
}

mtp_status mtp_verify_attn_workspace_size(const mtp_shape* shape, size_t* bytes) {
  const mtp_status st = check_shape(shape);
  if (st != MTP_OK) return st;
  if (bytes == nullptr) return MTP_ERR_NULL;
  const Plan pl = make_plan(*shape);
  *bytes = pl.ws_bytes;
  return MTP_OK;
}

mtp_status mtp_verify_attn_nested_workspace_size(const mtp_shape* shape, size_t* bytes) {
  const mtp_status st = check_shape(shape);
  if (st != MTP_OK) return st;
  if (bytes == nullptr) return MTP_ERR_NULL;
  const Plan pl = make_plan(*shape, true);
  *bytes = pl.ws_bytes;
  return MTP_OK;
}

}  // extern "C"

namespace {

enum Phase { kPartial = 1, kCombine = 2, kBoth = 3 };

struct Attn {
  Plan pl;
  AttnParams p;
  StreamParams sp;
};

mtp_status build_attn(const mtp_shape* shape, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_table, const int32_t* ctx_lens,
                      const void* k_new, const void* v_new, const uint8_t* mask_kind,
                      const int32_t* mask_ids, float* out, float* lse, void* workspace,
                      size_t workspace_bytes, Attn& a, bool nested = false) {
  const mtp_status st = check_shape(shape);
  if (st != MTP_OK) return st;
  const mtp_shape& s = *shape;
  if (nested && (s.D != 128 || s.dtype != MTP_BF16)) return MTP_ERR_UNSUPPORTED;
  if (s.B == 0) return MTP_OK;
  if (!q || (!nested && (!k_cache || !v_cache)) || !block_table || !ctx_lens || !k_new || !v_new ||
      !mask_kind || !mask_ids || !out || !workspace)
    return MTP_ERR_NULL;
  a.pl = make_plan(s, nested);
  const Plan& pl = a.pl;
  if (workspace_bytes < pl.ws_bytes || ((uintptr_t)workspace & 15) != 0)
    return MTP_ERR_WORKSPACE;
  AttnParams& p = a.p;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.ctx_lens = ctx_lens;
  p.k_new = k_new;
  p.v_new = v_new;
  p.mask_kind = mask_kind;
  p.mask_ids = mask_ids;
  p.part_acc = static_cast<float*>(workspace);
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ml_offset);
  p.out = out;
  p.lse = lse;
  p.B = s.B;
  p.W = s.W;
  p.Hq = s.Hq;
  p.Hkv = s.Hkv;
  p.g = pl.g;
  p.R = pl.R;
  p.nRB = pl.nRB;
  p.S = pl.S;
  p.n1 = pl.n1;
  p.S1 = pl.S1;
  p.max_splits = pl.max_splits;
  p.max_pages = s.max_pages_per_seq;
  p.num_pages = s.num_pages;
  p.max_ctx = s.max_ctx_len;
  p.lookback = s.seg_lookback;
  const float scale = s.scale > 0.f ? s.scale : 1.f / sqrtf((float)s.D);
  p.scale_log2 = scale * kLog2e;
  a.sp.seg_info = reinterpret_cast<int*>(static_cast<char*>(workspace) + pl.seg_offset);
  a.sp.nts = pl.nts;
  a.sp.nseg = pl.nseg;
  a.sp.rows_block = pl.rows_block;
  a.sp.h1 = pl.h1;
  a.sp.w_num = kFirstRoundNum;
  a.sp.w_den = kFirstRoundDen;
  a.sp.piece_rows = pl.piece_rows ? 1 : 0;
  return MTP_OK;
}

void launch_partial(const Attn& a, int D, int dtype, int B, hipStream_t strm,
                    const NestedAttn* na = nullptr) {
  const Plan& pl = a.pl;
  const AttnParams& p = a.p;
  const StreamParams& sp = a.sp;
  const dim3 block(256);
  const long items = (long)pl.max_splits * p.Hkv * pl.nRB;
  if (pl.kernel == kMfmaNestedStream) {
    const dim3 sgrid((unsigned)pl.G);
    const dim3 sblock(64 * pl.NR);
    if (na->kv8_recent == 0) {  // every committed key at 4 bits: base plane only
      if (pl.NR == 4) attn_partial_nested_stream<4, true><<<sgrid, sblock, 0, strm>>>(p, sp, *na);
      else if (pl.NR == 2) attn_partial_nested_stream<2, true><<<sgrid, sblock, 0, strm>>>(p, sp, *na);
      else attn_partial_nested_stream<1, true><<<sgrid, sblock, 0, strm>>>(p, sp, *na);
    } else {
      if (pl.NR == 4) attn_partial_nested_stream<4, false><<<sgrid, sblock, 0, strm>>>(p, sp, *na);
      else if (pl.NR == 2) attn_partial_nested_stream<2, false><<<sgrid, sblock, 0, strm>>>(p, sp, *na);
      else attn_partial_nested_stream<1, false><<<sgrid, sblock, 0, strm>>>(p, sp, *na);
    }
  } else if (pl.kernel == kMfmaNested) {
    const dim3 wgrid((unsigned)items, (unsigned)B);
    const dim3 wblock(64 * pl.NR);
    if (pl.NR == 4) attn_partial_nested_lds<1, 4><<<wgrid, wblock, 0, strm>>>(p, *na);
    else if (pl.NR == 2) attn_partial_nested_lds<1, 2><<<wgrid, wblock, 0, strm>>>(p, *na);
    else attn_partial_nested_lds<1, 1><<<wgrid, wblock, 0, strm>>>(p, *na);
  } else if (pl.kernel == kMfmaStream) {
    const dim3 sgrid((unsigned)pl.G);
    const dim3 sblock(64 * pl.NR);
    if (pl.RB == 2) attn_partial_stream<2, 4><<<sgrid, sblock, 0, strm>>>(p, sp);
    else if (pl.NR == 4) attn_partial_stream<1, 4><<<sgrid, sblock, 0, strm>>>(p, sp);
    else if (pl.NR == 2) attn_partial_stream<1, 2><<<sgrid, sblock, 0, strm>>>(p, sp);
    else attn_partial_stream<1, 1><<<sgrid, sblock, 0, strm>>>(p, sp);
  } else if (pl.kernel == kMfmaLds) {
    const dim3 wgrid((unsigned)items, (unsigned)B);
    const dim3 wblock(64 * pl.NR * pl.KS);
    if (pl.KS == 2 && pl.NR == 2) attn_partial_lds<1, 2, 2><<<wgrid, wblock, 0, strm>>>(p);
    else if (pl.KS == 2) attn_partial_lds<1, 1, 2><<<wgrid, wblock, 0, strm>>>(p);
    else if (pl.NR == 4) attn_partial_lds<1, 4><<<wgrid, wblock, 0, strm>>>(p);
    else if (pl.NR == 2) attn_partial_lds<1, 2><<<wgrid, wblock, 0, strm>>>(p);
    else attn_partial_lds<1, 1><<<wgrid, wblock, 0, strm>>>(p);
  } else {
    const dim3 grid((unsigned)((items + 3) / 4), (unsigned)B);
    if (pl.kernel == kMfmaDirect) {  // D = 64 only (D = 128 takes the LDS kernels)
      if (pl.RB == 4) attn_partial_mfma<64, 4><<<grid, block, 0, strm>>>(p);
      else if (pl.RB == 2) attn_partial_mfma<64, 2><<<grid, block, 0, strm>>>(p);
      else attn_partial_mfma<64, 1><<<grid, block, 0, strm>>>(p);
    } else if (dtype == MTP_F32) {
      if (D == 128) attn_partial_valu<float, 128><<<grid, block, 0, strm>>>(p);
      else attn_partial_valu<float, 64><<<grid, block, 0, strm>>>(p);
    } else {
      if (D == 128) attn_partial_valu<uint16_t, 128><<<grid, block, 0, strm>>>(p);
      else attn_partial_valu<uint16_t, 64><<<grid, block, 0, strm>>>(p);
    }
  }
}

// Output rows one combine wave takes: four (one per 16-lane group) for the
// stream layout with few pieces per segment and for split layouts with few
// splits, one otherwise.  `finish`: the step's finish launch (grouped for
// the stream layout only).
bool grouped_combine(const AttnParams& p, const Plan& pl, bool finish) {
  if (stream_layout(pl.kernel)) return !pl.piece_rows;
  return !finish && grouped_split_combine(pl.max_splits, (long)p.B * p.W * p.Hq);
}
int combine_rows_per_wave(const AttnParams& p, const Plan& pl, bool finish) {
  return grouped_combine(p, pl, finish) ? 4 : 1;
}

// Workgroups of a combine launch with `waves` combine waves per workgroup.
// Grouped-combine waves loop over their rows, so at most `cap` workgroups.
unsigned combine_blocks(const AttnParams& p, const Plan& pl, bool finish, int waves, long cap) {
  const size_t per = (size_t)waves * combine_rows_per_wave(p, pl, finish);
  const long n = (long)(((size_t)p.B * p.W * p.Hq + per - 1) / per);
  return (unsigned)(grouped_combine(p, pl, finish) ? std::max(1L, std::min(n, cap)) : n);
}

// Compute units the combine workgroups of the step's finish launch may take:
// those the B acceptance workgroups leave free; with the per-split layout
// (one row per wave) at most kFinishSplitCUs of them when the acceptance
// reduces the logits rows itself: its chain of dependent loads runs beside
// the combine, and fewer combine workgroups in flight leave its loads less
// to queue behind (llama3_8b_tree step 29.9 -> 29.3 us).  When the partial
// launch found the targets (step_target_prologue) the acceptance reads W
// words instead, and the combine takes every free CU (llama3_8b_tree step
// 24.7 -> 24.0 us).
constexpr long kFinishSplitCUs = 128;
long finish_combine_cus(const AttnParams& p, const Plan& pl) {
  // More sequences than half the compute units: their acceptance workgroups
  // occupy the chip for a while anyway, and subtracting them would leave the
  // (looping) combine a handful of workgroups for the whole batch; it keeps
  // one workgroup per compute unit instead, dispatched behind them.
  const long free_cus = p.B <= kCUs / 2 ? (long)kCUs - p.B : (long)kCUs;
  if (grouped_combine(p, pl, true) || p.logits != nullptr) return free_cus;
  return std::min(kFinishSplitCUs, free_cus);
}

// Combine waves per workgroup of the step's finish launch.  Its workgroups
// have kAcceptThreads threads, one per compute unit at a time; the rows are
// spread so that the combine workgroups and the B acceptance workgroups fit
// on the compute units together (few rows: one combine wave per workgroup,
// so that they spread over as many compute units as possible).
int finish_combine_waves(const AttnParams& p, const Plan& pl) {
  const int rpw = combine_rows_per_wave(p, pl, true);
  const long waves = ((long)p.B * p.W * p.Hq + rpw - 1) / rpw;
  const long cus = finish_combine_cus(p, pl);
  const long per = (waves + cus - 1) / cus;
  return (int)std::min<long>(kAcceptThreads / kWave, std::max(1L, per));
}

void launch_combine(const Attn& a, int D, hipStream_t strm) {
  const dim3 cgrid(combine_blocks(a.p, a.pl, false, 4, 4L * kCUs)), block(256);
  if (stream_layout(a.pl.kernel)) attn_combine<128, true><<<cgrid, block, 0, strm>>>(a.p, a.sp);
  else if (D == 128) attn_combine<128, false><<<cgrid, block, 0, strm>>>(a.p, a.sp);
  else attn_combine<64, false><<<cgrid, block, 0, strm>>>(a.p, a.sp);
}

mtp_status verify_attn_phases(int phases, const mtp_shape* shape, const void* q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* ctx_lens,
                              const void* k_new, const void* v_new, const uint8_t* mask_kind,
                              const int32_t* mask_ids, float* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream) {
  Attn a;
  const mtp_status st = build_attn(shape, q, k_cache, v_cache, block_table, ctx_lens, k_new, v_new,
                                   mask_kind, mask_ids, out, lse, workspace, workspace_bytes, a);
  if (st != MTP_OK || shape->B == 0) return st;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  if (phases & kPartial) launch_partial(a, shape->D, shape->dtype, shape->B, strm);
  if (phases & kCombine) launch_combine(a, shape->D, strm);
  return launch_status();
}

}  // namespace

extern "C" {

#define MTPV_ATTN_ARGS                                                                       \
  const mtp_shape *shape, const void *q, const void *k_cache, const void *v_cache,         \
      const int32_t *block_table, const int32_t *ctx_lens, const void *k_new,              \
      const void *v_new, const uint8_t *mask_kind, const int32_t *mask_ids, float *out,    \
      float *lse, void *workspace, size_t workspace_bytes, void *stream
#define MTPV_ATTN_PASS                                                                      \
  shape, q, k_cache, v_cache, block_table, ctx_lens, k_new, v_new, mask_kind, mask_ids, out, \
      lse, workspace, workspace_bytes, stream

mtp_status mtp_verify_attn(MTPV_ATTN_ARGS) { return verify_attn_phases(kBoth, MTPV_ATTN_PASS); }

mtp_status mtp_verify_attn_partial(MTPV_ATTN_ARGS) {
  return verify_attn_phases(kPartial, MTPV_ATTN_PASS);
}

mtp_status mtp_verify_attn_combine(MTPV_ATTN_ARGS) {
  return verify_attn_phases(kCombine, MTPV_ATTN_PASS);
}

static mtp_status fill_accept(const mtp_shape* shape, const float* logits, int32_t V,
                              const int32_t* draft_ids, const uint8_t* mask_kind,
                              const int32_t* mask_ids, int32_t* accept_len, int32_t* accept_path,
                              int32_t* bonus_id, AcceptParams& ap) {
  if (shape == nullptr) return MTP_ERR_NULL;
  if (shape->B < 0 || shape->W < 1 || shape->W > MTP_MAX_W || V < 1) return MTP_ERR_SHAPE;
  if (shape->B > 0 && (!logits || !draft_ids || !mask_kind || !mask_ids || !accept_len ||
                       !accept_path || !bonus_id))
    return MTP_ERR_NULL;
  ap.logits = logits;
  ap.draft_ids = draft_ids;
  ap.mask_kind = mask_kind;
  ap.mask_ids = mask_ids;
  ap.accept_len = accept_len;
  ap.accept_path = accept_path;
  ap.bonus_id = bonus_id;
  ap.B = shape->B;
  ap.W = shape->W;
  ap.V = V;
  return MTP_OK;
}

static mtp_status fill_commit(const mtp_shape* shape, const void* k_new, const void* v_new,
                              const int32_t* accept_len, const int32_t* accept_path,
                              const int32_t* block_table, const int32_t* ctx_lens_in,
                              int32_t* ctx_lens_out, int32_t skip_root, void* k_cache,
                              void* v_cache, bool fused, CommitParams& cp) {
  const mtp_status st = check_shape(shape);
  if (st != MTP_OK) return st;
  if (shape->B > 0 &&
      (!k_new || !v_new || !block_table || !ctx_lens_in || !ctx_lens_out || !k_cache || !v_cache ||
       (!fused && (!accept_len || !accept_path))))
    return MTP_ERR_NULL;
  const int elem = shape->dtype == MTP_F32 ? 4 : 2;
  cp.k_new = k_new;
  cp.v_new = v_new;
  cp.accept_len = accept_len;
  cp.accept_path = accept_path;
  cp.block_table = block_table;
  cp.ctx_in = ctx_lens_in;
  cp.ctx_out = ctx_lens_out;
  cp.k_cache = k_cache;
  cp.v_cache = v_cache;
  cp.skip_root = skip_root ? 1 : 0;
  cp.W = shape->W;
  cp.max_pages = shape->max_pages_per_seq;
  cp.num_pages = shape->num_pages;
  cp.row_bytes = shape->Hkv * shape->D * elem;
  return MTP_OK;
}

mtp_status mtp_accept(const mtp_shape* shape, const float* logits, int32_t V,
                      const int32_t* draft_ids, const uint8_t* mask_kind,
                      const int32_t* mask_ids, int32_t* accept_len, int32_t* accept_path,
                      int32_t* bonus_id, void* stream) {
  AcceptParams ap;
  const mtp_status st = fill_accept(shape, logits, V, draft_ids, mask_kind, mask_ids, accept_len,
                                    accept_path, bonus_id, ap);
  if (st != MTP_OK || shape->B == 0) return st;
  accept_kernel<<<dim3(shape->B), dim3(kAcceptThreads), 0, static_cast<hipStream_t>(stream)>>>(ap);
  return launch_status();
}

mtp_status mtp_accept_hybrid(const mtp_shape* shape, const float* draft_logits,
                             const float* logits, int32_t V, const int32_t* draft_ids,
                             const uint8_t* mask_kind, const int32_t* mask_ids, float tau,
                             int32_t min_prefix, int32_t* accept_len, int32_t* accept_path,
                             int32_t* bonus_id, int32_t* conf_len, void* stream) {
  if (shape == nullptr) return MTP_ERR_NULL;
  if (shape->B > 0 && (!draft_logits || !conf_len)) return MTP_ERR_NULL;
  if (tau != tau) return MTP_ERR_SHAPE;
  AcceptParams ap;
  // the greedy checks, with a stand-in for the optional verifier logits
  const mtp_status st = fill_accept(shape, logits != nullptr ? logits : draft_logits, V, draft_ids,
                                    mask_kind, mask_ids, accept_len, accept_path, bonus_id, ap);
  if (st != MTP_OK || shape->B == 0) return st;
  ap.logits = logits;
  HybridParams hp;
  hp.draft_logits = draft_logits;
  hp.conf_len = conf_len;
  hp.tau = tau;
  hp.min_prefix = min_prefix;
  const int ntask = (shape->W - 1) + (logits != nullptr ? shape->W : 0);
  const int threads = kWave * std::min(16, std::max(1, ntask));
  accept_hybrid_kernel<<<dim3(shape->B), dim3(threads), 0, static_cast<hipStream_t>(stream)>>>(ap, hp);
  return launch_status();
}

mtp_status mtp_kv_commit(const mtp_shape* shape, const void* k_new, const void* v_new,
                         const int32_t* accept_len, const int32_t* accept_path,
                         const int32_t* block_table, const int32_t* ctx_lens_in,
                         int32_t* ctx_lens_out, int32_t skip_root, void* k_cache,
                         void* v_cache, void* stream) {
  CommitParams cp;
  const mtp_status st = fill_commit(shape, k_new, v_new, accept_len, accept_path, block_table,
                                    ctx_lens_in, ctx_lens_out, skip_root, k_cache, v_cache, false,
                                    cp);
  if (st != MTP_OK || shape->B == 0) return st;
  commit_kernel<<<dim3(shape->B), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(cp);
  return launch_status();
}

mtp_status mtp_accept_commit(const mtp_shape* shape, const float* logits, int32_t V,
                             const int32_t* draft_ids, const uint8_t* mask_kind,
                             const int32_t* mask_ids, int32_t* accept_len,
                             int32_t* accept_path, int32_t* bonus_id, const void* k_new,
                             const void* v_new, const int32_t* block_table,
                             const int32_t* ctx_lens_in, int32_t* ctx_lens_out,
                             int32_t skip_root, void* k_cache, void* v_cache, void* stream) {
  AcceptParams ap;
  mtp_status st = fill_accept(shape, logits, V, draft_ids, mask_kind, mask_ids, accept_len,
                              accept_path, bonus_id, ap);
  if (st != MTP_OK) return st;
  CommitParams cp;
  st = fill_commit(shape, k_new, v_new, accept_len, accept_path, block_table, ctx_lens_in,
                   ctx_lens_out, skip_root, k_cache, v_cache, true, cp);
  if (st != MTP_OK || shape->B == 0) return st;
  accept_commit_kernel<<<dim3(shape->B), dim3(kAcceptThreads), 0, static_cast<hipStream_t>(stream)>>>(ap, cp);
  return launch_status();
}

mtp_status mtp_verify_step(const mtp_shape* shape, const void* q, void* k_cache, void* v_cache,
                           const int32_t* block_table, const int32_t* ctx_lens_in,
                           const void* k_new, const void* v_new, const uint8_t* mask_kind,
                           const int32_t* mask_ids, const float* logits, int32_t V,
                           const int32_t* draft_ids, float* out, float* lse,
                           int32_t* accept_len, int32_t* accept_path, int32_t* bonus_id,
                           int32_t* ctx_lens_out, int32_t skip_root, void* workspace,
                           size_t workspace_bytes, void* stream) {
  Attn a;
  mtp_status st = build_attn(shape, q, k_cache, v_cache, block_table, ctx_lens_in, k_new, v_new,
                             mask_kind, mask_ids, out, lse, workspace, workspace_bytes, a);
  if (st != MTP_OK) return st;
  AcceptParams ap;
  st = fill_accept(shape, logits, V, draft_ids, mask_kind, mask_ids, accept_len, accept_path,
                   bonus_id, ap);
  if (st != MTP_OK) return st;
  CommitParams cp;
  st = fill_commit(shape, k_new, v_new, accept_len, accept_path, block_table, ctx_lens_in,
                   ctx_lens_out, skip_root, k_cache, v_cache, true, cp);
  if (st != MTP_OK || shape->B == 0) return st;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  if (ctx_lens_out != ctx_lens_in && step_target_prologue(a.pl, *shape, logits, V)) {
    // the partial launch finds the row targets; the acceptance reads them
    int32_t* tgt = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + a.pl.tgt_offset);
    a.p.logits = logits;
    a.p.tgt = tgt;
    a.p.V = V;
    ap.tgt = tgt;
  }
  launch_partial(a, shape->D, shape->dtype, shape->B, strm);
  if (ctx_lens_out == ctx_lens_in) {  // the combine reads what the commit writes: serialise
    launch_combine(a, shape->D, strm);
    accept_commit_kernel<<<dim3(shape->B), dim3(kAcceptThreads), 0, strm>>>(ap, cp);
  } else {
    const int crows = finish_combine_waves(a.p, a.pl);
    const dim3 fgrid((unsigned)shape->B +
                     combine_blocks(a.p, a.pl, true, crows, finish_combine_cus(a.p, a.pl))),
        block(kAcceptThreads);
    if (stream_layout(a.pl.kernel))
      finish_kernel<128, true><<<fgrid, block, 0, strm>>>(a.p, a.sp, ap, cp, crows);
    else if (shape->D == 128)
      finish_kernel<128, false><<<fgrid, block, 0, strm>>>(a.p, a.sp, ap, cp, crows);
    else
      finish_kernel<64, false><<<fgrid, block, 0, strm>>>(a.p, a.sp, ap, cp, crows);
  }
  return launch_status();
}

}  // extern "C"

// ---- the step without a caller workspace ----------------------------------
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the step's
// split-K partials go to this file-scope device array instead of a caller
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, never
// the device memory: host code uses only the address hipGetSymbolAddress
// returns on each device, taken once per device with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device

mtp_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MTP_ERR_HIP;
  if (dev >= kMaxScratchDevices) return MTP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return MTP_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MTP_OK;
}

}  // namespace

extern "C" {

mtp_status mtp_verify_step_noalloc(const mtp_shape* shape, const void* q, void* k_cache,
                                   void* v_cache, const int32_t* block_table,
                                   const int32_t* ctx_lens_in, const void* k_new,
                                   const void* v_new, const uint8_t* mask_kind,
                                   const int32_t* mask_ids, const float* logits, int32_t V,
                                   const int32_t* draft_ids, float* out, float* lse,
                                   int32_t* accept_len, int32_t* accept_path, int32_t* bonus_id,
                                   int32_t* ctx_lens_out, int32_t skip_root, void* stream) {
  // the size check comes first and needs no device
  const mtp_status st = check_shape(shape);
  if (st != MTP_OK) return st;
  const Plan pl = make_plan(*shape);
  if (pl.ws_bytes > kScratchBytes) return MTP_ERR_SCRATCH;
  void* ws = nullptr;
  if (shape->B > 0) {
    const mtp_status ss = scratch_of_current_device(&ws);
    if (ss != MTP_OK) return ss;
  }
  // Nothing in the scratch needs to start at zero: the partial launch writes
  // every partial and segment record the combine reads.
  return mtp_verify_step(shape, q, k_cache, v_cache, block_table, ctx_lens_in, k_new, v_new,
                         mask_kind, mask_ids, logits, V, draft_ids, out, lse, accept_len,
                         accept_path, bonus_id, ctx_lens_out, skip_root, ws,
                         ws != nullptr ? kScratchBytes : 0, stream);
}

static bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

// Checks the planes a nested-cache call needs (refinement planes unless
// `base_only`): present and 16-byte aligned.
static mtp_status check_nested(const mtp_nested_kv* kv, bool base_only) {
  if (kv == nullptr || !kv->k_base || !kv->k_scale || !kv->v_base || !kv->v_scale) return MTP_ERR_NULL;
  if (!base_only && (!kv->k_ref || !kv->v_ref)) return MTP_ERR_NULL;
  if (!aligned16(kv->k_base) || !aligned16(kv->k_scale) || !aligned16(kv->v_base) ||
      !aligned16(kv->v_scale) || (!base_only && (!aligned16(kv->k_ref) || !aligned16(kv->v_ref))))
    return MTP_ERR_SHAPE;
  return MTP_OK;
}

static mtp_status verify_attn_nested_phases(int phases, const mtp_shape* shape, const void* q,
                                            const mtp_nested_kv* kv, const int32_t* block_table,
                                            const int32_t* ctx_lens, const void* k_new,
                                            const void* v_new, const uint8_t* mask_kind,
                                            const int32_t* mask_ids, int32_t kv8_recent,
                                            float* out, float* lse, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  Attn a;
  mtp_status st = build_attn(shape, q, nullptr, nullptr, block_table, ctx_lens, k_new, v_new,
                             mask_kind, mask_ids, out, lse, workspace, workspace_bytes, a, true);
  if (st != MTP_OK || shape->B == 0) return st;
  if (kv8_recent < -1) return MTP_ERR_SHAPE;
  st = check_nested(kv, kv8_recent == 0);
  if (st != MTP_OK) return st;
  NestedAttn na;
  na.kv = *kv;
  na.kv8_recent = kv8_recent;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  if (phases & kPartial) launch_partial(a, shape->D, shape->dtype, shape->B, strm, &na);
  if (phases & kCombine) launch_combine(a, shape->D, strm);
  return launch_status();
}

#define MTPV_NESTED_ARGS                                                                     \
  const mtp_shape *shape, const void *q, const mtp_nested_kv *kv, const int32_t *block_table, \
      const int32_t *ctx_lens, const void *k_new, const void *v_new,                          \
      const uint8_t *mask_kind, const int32_t *mask_ids, int32_t kv8_recent, float *out,      \
      float *lse, void *workspace, size_t workspace_bytes, void *stream
#define MTPV_NESTED_PASS                                                                      \
  shape, q, kv, block_table, ctx_lens, k_new, v_new, mask_kind, mask_ids, kv8_recent, out, lse, \
      workspace, workspace_bytes, stream

mtp_status mtp_verify_attn_nested(MTPV_NESTED_ARGS) {
  return verify_attn_nested_phases(kBoth, MTPV_NESTED_PASS);
}

mtp_status mtp_verify_attn_nested_partial(MTPV_NESTED_ARGS) {
  return verify_attn_nested_phases(kPartial, MTPV_NESTED_PASS);
}

mtp_status mtp_verify_attn_nested_combine(MTPV_NESTED_ARGS) {
  return verify_attn_nested_phases(kCombine, MTPV_NESTED_PASS);
}

mtp_status mtp_kv_quantize(const mtp_shape* shape, const void* k_rows, const void* v_rows,
                           int32_t n_rows, const int32_t* slots, const mtp_nested_kv* kv,
                           void* stream) {
  const mtp_status st = check_shape(shape);
  if (st != MTP_OK) return st;
  if (n_rows < 0) return MTP_ERR_SHAPE;
  if (n_rows == 0) return MTP_OK;
  if (!k_rows || !v_rows || !slots) return MTP_ERR_NULL;
  const mtp_status sn = check_nested(kv, false);
  if (sn != MTP_OK) return sn;
  QuantizeParams p;
  p.k_rows = k_rows;
  p.v_rows = v_rows;
  p.slots = slots;
  p.kv = *kv;
  p.n = n_rows;
  p.Hkv = shape->Hkv;
  p.D = shape->D;
  p.dtype = shape->dtype;
  p.num_pages = shape->num_pages;
  const long waves = (long)n_rows * shape->Hkv * 2;
  if ((waves + 3) / 4 > 0x7fffffffL) return MTP_ERR_SHAPE;
  kv_quantize_kernel<<<dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       static_cast<hipStream_t>(stream)>>>(p);
  return launch_status();
}

mtp_status mtp_kv_commit_nested(const mtp_shape* shape, const void* k_new, const void* v_new,
                                const int32_t* accept_len, const int32_t* accept_path,
                                const int32_t* block_table, const int32_t* ctx_lens_in,
                                int32_t* ctx_lens_out, int32_t skip_root, const mtp_nested_kv* kv,
                                void* stream) {
  NestedCommitParams np;
  // the plain commit's checks, with the planes standing in for the cache
  mtp_status st = fill_commit(shape, k_new, v_new, accept_len, accept_path, block_table,
                              ctx_lens_in, ctx_lens_out, skip_root,
                              kv != nullptr ? kv->k_base : nullptr,
                              kv != nullptr ? kv->v_base : nullptr, false, np.c);
  if (st != MTP_OK || shape->B == 0) return st;
  st = check_nested(kv, false);
  if (st != MTP_OK) return st;
  np.kv = *kv;
  np.Hkv = shape->Hkv;
  np.D = shape->D;
  np.dtype = shape->dtype;
  commit_nested_kernel<<<dim3(shape->B), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(np);
  return launch_status();
}

static mtp_status check_tree(int32_t B, int32_t K, int32_t V, int32_t W, int32_t n_mask) {
  if (B < 0 || B > 65535 || K < 1 || K > kTreeMaxK || V < 1 || V > kTreeMaxV || W < 1 ||
      W > MTP_MAX_W || n_mask < 0 || n_mask > W - 1)
    return MTP_ERR_SHAPE;
  return MTP_OK;
}

static size_t tree_list_bytes(int32_t B, int32_t K, int32_t W, int32_t n_mask) {
  return (size_t)B * K * (size_t)(W - n_mask) * 4;  // one int32 or fp32 array
}

mtp_status mtp_build_tree_workspace_size(int32_t B, int32_t K, int32_t V, int32_t W,
                                         int32_t n_mask, size_t* bytes) {
  const mtp_status st = check_tree(B, K, V, W, n_mask);
  if (st != MTP_OK) return st;
  if (bytes == nullptr) return MTP_ERR_NULL;
  *bytes = 2 * ((tree_list_bytes(B, K, W, n_mask) + 255) & ~(size_t)255);
  return MTP_OK;
}

mtp_status mtp_build_tree(int32_t B, int32_t K, int32_t V, int32_t W, int32_t n_mask,
                          const float* probs, const int32_t* root_token, float min_cum_prob,
                          int32_t* draft_ids, int32_t* parents, int32_t* depth,
                          int32_t* n_nodes, void* workspace, size_t workspace_bytes,
                          void* stream) {
  mtp_status st = check_tree(B, K, V, W, n_mask);
  if (st != MTP_OK) return st;
  if (min_cum_prob != min_cum_prob) return MTP_ERR_SHAPE;
  if (B == 0) return MTP_OK;
  if (!probs || !root_token || !draft_ids || !parents || !depth || !n_nodes || !workspace)
    return MTP_ERR_NULL;
  const size_t half = (tree_list_bytes(B, K, W, n_mask) + 255) & ~(size_t)255;
  if (workspace_bytes < 2 * half || ((uintptr_t)workspace & 15) != 0) return MTP_ERR_WORKSPACE;
  TreeParams p;
  p.probs = probs;
  p.root = root_token;
  p.draft = draft_ids;
  p.parent = parents;
  p.depth = depth;
  p.n_nodes = n_nodes;
  p.list_tok = static_cast<int*>(workspace);
  p.list_prb = reinterpret_cast<float*>(static_cast<char*>(workspace) + half);
  p.min_cum_prob = min_cum_prob;
  p.B = B;
  p.K = K;
  p.V = V;
  p.W = W;
  p.n_mask = n_mask;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  if (W - 1 - n_mask > 0)
    tree_lists_kernel<<<dim3(K, B), dim3(kTreeListThreads), 0, strm>>>(p);
  tree_build_kernel<<<dim3(B), dim3(256), 0, strm>>>(p);
  return launch_status();
}

mtp_status mtp_block_positions(const mtp_shape* shape, const int32_t* ctx_lens,
                               const uint8_t* mask_kind, const int32_t* mask_ids,
                               int32_t* positions, void* stream) {
  if (shape == nullptr) return MTP_ERR_NULL;
  if (shape->B < 0 || shape->B > 65535 * 4 || shape->W < 1 || shape->W > MTP_MAX_W)
    return MTP_ERR_SHAPE;
  if (shape->B == 0) return MTP_OK;
  if (!ctx_lens || !mask_kind || !mask_ids || !positions) return MTP_ERR_NULL;
  positions_kernel<<<dim3((unsigned)((shape->B + 3) / 4)), dim3(256), 0,
                     static_cast<hipStream_t>(stream)>>>(ctx_lens, mask_kind, mask_ids, positions,
                                                         shape->B, shape->W);
  return launch_status();
}

mtp_status mtp_check_commit_slots(const mtp_shape* shape, const int32_t* block_table,
                                  const int32_t* ctx_lens, int32_t* bad_seq) {
  if (shape == nullptr) return MTP_ERR_NULL;
  const mtp_shape& s = *shape;
  if (s.B < 0 || s.W < 1 || s.W > MTP_MAX_W || s.num_pages < 0 || s.max_pages_per_seq < 0)
    return MTP_ERR_SHAPE;
  if (bad_seq != nullptr) *bad_seq = -1;
  if (s.B == 0) return MTP_OK;
  if (ctx_lens == nullptr || (s.max_pages_per_seq > 0 && block_table == nullptr))
    return MTP_ERR_NULL;
  const int32_t bad = first_commit_conflict(s.B, s.W, s.num_pages, s.max_pages_per_seq,
                                            block_table, ctx_lens);
  if (bad_seq != nullptr) *bad_seq = bad;
  return bad < 0 ? MTP_OK : MTP_ERR_CONFLICT;
}

mtp_status mtp_get_device_status(uint32_t* bits, int32_t clear) {
  if (bits == nullptr) return MTP_ERR_NULL;
  if (hipDeviceSynchronize() != hipSuccess) return MTP_ERR_HIP;
  unsigned v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_status), sizeof(v), 0, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return MTP_ERR_HIP;
  *bits = v;
  if (clear) {
    const unsigned zero = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_status), &zero, sizeof(zero), 0, hipMemcpyHostToDevice) !=
        hipSuccess)
      return MTP_ERR_HIP;
  }
  return MTP_OK;
}

}  // extern "C"
