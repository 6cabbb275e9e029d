// C ABI of the gfx950 attention library: argument validation, workspace sizing
// and kernel selection.  Every check runs before the first HIP call, so a
// rejected call leaves no work on the stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa_gfx950.h"
#include "fa_internal.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxOffsetBytes = (int64_t)1 << 31;  // 32-bit buffer offsets

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Shape {
  bool varlen;
  int batch, heads, d;
  int max_q, max_k;
  int total_q, total_k;  // fixed length: batch * seqlen
  const int32_t* cu_q;
  const int32_t* cu_k;
};

// Shared validation of the geometry fields of fa_fwd_args / fa_bwd_args.
fa_status check_shape(int batch, int seqlen_q, int seqlen_k, int heads, int d, const int32_t* cu_q,
                      const int32_t* cu_k, int max_q, int max_k, int total_q, int total_k, int causal,
                      float scale, Shape* out) {
  if (batch < 0 || heads <= 0 || d <= 0) return FA_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARGUMENT;
  // The kernels take the row maximum over the raw scores and fold the scale into the
  // exponent, which needs scale > 0 (scale = 0 would also turn a hidden key's -inf
  // score times 0 into NaN).
  if (!(scale > 0.0f)) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARGUMENT;
  Shape s{};
  s.batch = batch;
  s.heads = heads;
  s.d = d;
  if (cu_q != nullptr) {
    s.varlen = true;
    if (max_q < 0 || total_q < 0) return FA_ERR_INVALID_ARGUMENT;
    if (cu_k == nullptr) {
      cu_k = cu_q;
      max_k = max_q;
      total_k = total_q;
    }
    if (max_k < 0 || total_k < 0) return FA_ERR_INVALID_ARGUMENT;
    if (((uintptr_t)cu_q & 3u) || ((uintptr_t)cu_k & 3u)) return FA_ERR_INVALID_ARGUMENT;
    s.max_q = max_q;
    s.max_k = max_k;
    s.total_q = total_q;
    s.total_k = total_k;
  } else {
    if (cu_k != nullptr) return FA_ERR_INVALID_ARGUMENT;
    if (seqlen_q < 0 || seqlen_k < 0) return FA_ERR_INVALID_ARGUMENT;
    s.varlen = false;
    s.max_q = seqlen_q;
    s.max_k = seqlen_k;
    if ((int64_t)batch * seqlen_q > INT32_MAX || (int64_t)batch * seqlen_k > INT32_MAX) return FA_ERR_UNSUPPORTED;
    s.total_q = batch * seqlen_q;
    s.total_k = batch * seqlen_k;
  }
  if ((s.max_q + 63) / 64 > fa::kSchedMaxCost || (s.max_k + 63) / 64 > fa::kSchedMaxCost) return FA_ERR_UNSUPPORTED;
  if (batch > 65535 || heads > 65535) return FA_ERR_UNSUPPORTED;  // grid dimensions of per-sequence kernels
  s.cu_q = cu_q;
  s.cu_k = cu_k;
  *out = s;
  return FA_OK;
}

// Strides: D contiguous is implied; S/H (and B for fixed length) must keep 16-byte
// alignment; every row a kernel may touch (including a tile's padding rows) must
// stay within 32-bit byte offsets of the sequence base.
fa_status check_tensor(const void* ptr, const int64_t st[3], const Shape& s, int rows_max, int elem_bytes) {
  if (ptr == nullptr) return FA_ERR_INVALID_ARGUMENT;
  if (!aligned16(ptr)) return FA_ERR_INVALID_ARGUMENT;
  const int64_t sb = st[0], ss = st[1], sh = st[2];
  if (ss < s.d || sh < 0 || sb < 0) return FA_ERR_INVALID_ARGUMENT;
  const int64_t al = 16 / elem_bytes;
  if (ss % al || sh % al || (!s.varlen && sb % al)) return FA_ERR_INVALID_ARGUMENT;
  if ((int64_t)(rows_max + 256) * ss * elem_bytes + (int64_t)s.d * elem_bytes >= kMaxOffsetBytes) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int fwd_max_items(const Shape& s, int tile_rows) { return (s.total_q + tile_rows - 1) / tile_rows + s.batch; }

struct FwdChoice {
  int poly, tau, qt, splits;  // splits <= 0: chosen from the shape
};

constexpr int kMaxKeySplits = 64;

fa_status pick_tuning(const fa_fwd_tuning* t, FwdChoice* c) {
  c->poly = 0;
  c->tau = 8;
  c->qt = 2;
  c->splits = 0;
  if (t == nullptr) return FA_OK;
  if (t->key_splits > kMaxKeySplits) return FA_ERR_UNSUPPORTED;
  c->splits = t->key_splits > 0 ? t->key_splits : 0;
  if (t->exp2_poly_per16 >= 0) c->poly = t->exp2_poly_per16;
  if (t->rescale_threshold_log2 >= 0) c->tau = t->rescale_threshold_log2;
  if (t->q_tiles_per_workgroup >= 0) c->qt = t->q_tiles_per_workgroup;
  if (c->qt != 1 && c->qt != 2) return FA_ERR_UNSUPPORTED;
  if (c->tau == 8 && (c->poly == 0 || c->poly == 2 || c->poly == 4)) return FA_OK;
  if (c->tau == 0 && c->poly == 0) return FA_OK;
  return FA_ERR_UNSUPPORTED;
}

// The exp2 split shares 2 and 4 and the eager threshold are compiled for head_dim 128
// and fixed-length batches only (they exist to be measured against the default).
fa_status check_variant(const Shape& s, const FwdChoice& c) {
  if (c.poly == 0 && c.tau == 8) return FA_OK;
  return (s.d == 128 && !s.varlen) ? FA_OK : FA_ERR_UNSUPPORTED;
}

fa_status check_fwd(const fa_fwd_args* a, Shape* s) {
  if (a == nullptr) return FA_ERR_INVALID_ARGUMENT;
  fa_status st = check_shape(a->batch, a->seqlen_q, a->seqlen_k, a->num_heads, a->head_dim, a->cu_seqlens_q,
                             a->cu_seqlens_k, a->max_seqlen_q, a->max_seqlen_k, a->total_q, a->total_k, a->causal,
                             a->softmax_scale, s);
  if (st != FA_OK) return st;
  if ((st = check_tensor(a->q, a->q_stride, *s, s->max_q, 2)) != FA_OK) return st;
  if ((st = check_tensor(a->k, a->k_stride, *s, s->max_k, 2)) != FA_OK) return st;
  if ((st = check_tensor(a->v, a->v_stride, *s, s->max_k, 2)) != FA_OK) return st;
  if (a->o_dtype != FA_DTYPE_BF16 && a->o_dtype != FA_DTYPE_F32) return FA_ERR_INVALID_ARGUMENT;
  if ((st = check_tensor(a->o, a->o_stride, *s, s->max_q, a->o_dtype == FA_DTYPE_F32 ? 4 : 2)) != FA_OK) return st;
  if (a->lse == nullptr || ((uintptr_t)a->lse & 3u)) return FA_ERR_INVALID_ARGUMENT;
  return FA_OK;
}

// Key chunks for the split forward, when the query tiles alone (at 128 rows) leave
// the GPU short of work: about 512 workgroups in all (two per compute unit; more
// chunks only add per-chunk start, store and merge costs to a pass bound by reading K
// and V), each chunk spanning at least 32 key tiles of 64 — 16 where chunks that long
// would leave fewer workgroups than compute units.
int fwd_key_splits(const Shape& s, const FwdChoice& c) {
  if (c.splits > 0) return c.splits;
  const int64_t items = (int64_t)(s.varlen ? fwd_max_items(s, fa::kFwdTileRows)
                                           : (s.max_q + fa::kFwdTileRows - 1) / fa::kFwdTileRows * s.batch) *
                        s.heads;
  const int key_tiles = (s.max_k + fa::kFwdBlockN - 1) / fa::kFwdBlockN;
  if (items >= 512 || key_tiles < 32) return 1;
  const int want = (int)((512 + items - 1) / items);
  const int longest = items * (key_tiles / 32) >= 256 ? key_tiles / 32 : key_tiles / 16;
  return std::max(1, std::min({want, longest, kMaxKeySplits}));
}

// Forward workspace: [work list (variable length)] [partial LSE] [partial O]
// [fp16 copy of V: H x total_k x D] [per-tile exponents of the copy: H x total_k int32]
struct FwdWs {
  size_t lse_off, o_off, v16_off, vexp_off, total;
};

FwdWs fwd_ws_layout(const Shape& s, int tile_rows, int splits) {
  FwdWs w{};
  size_t off = s.varlen ? round_up(sizeof(int32_t) * (1 + 2 * (size_t)fwd_max_items(s, tile_rows))) : 0;
  if (splits > 1) {
    const size_t rows = (size_t)splits * s.heads * s.total_q;
    w.lse_off = off;
    off += round_up(rows * sizeof(float));
    w.o_off = off;
    off += round_up(rows * s.d * sizeof(float));
  }
  if (splits <= 1) {  // the key-split path reads V itself
    const size_t krows = (size_t)s.heads * s.total_k;
    w.v16_off = off;
    off += round_up(krows * s.d * sizeof(uint16_t));
    w.vexp_off = off;
    off += round_up(krows * sizeof(int32_t));
  }
  w.total = off;
  return w;
}

fa::FwdParams make_fwd_params(const fa_fwd_args* a, const Shape& s) {
  fa::FwdParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.q_sb = a->q_stride[0]; p.q_ss = a->q_stride[1]; p.q_sh = a->q_stride[2];
  p.k_sb = a->k_stride[0]; p.k_ss = a->k_stride[1]; p.k_sh = a->k_stride[2];
  p.v_sb = a->v_stride[0]; p.v_ss = a->v_stride[1]; p.v_sh = a->v_stride[2];
  p.o_sb = a->o_stride[0]; p.o_ss = a->o_stride[1]; p.o_sh = a->o_stride[2];
  p.o_f32 = a->o_dtype == FA_DTYPE_F32 ? 1 : 0;
  p.batch = s.batch;
  p.seqlen_q = s.max_q;
  p.seqlen_k = s.max_k;
  p.heads = s.heads;
  p.cu_q = s.cu_q;
  p.cu_k = s.cu_k;
  p.total_q = s.total_q;
  p.total_k = s.total_k;
  p.scale = a->softmax_scale;
  p.scale_log2 = (float)((double)a->softmax_scale * 1.4426950408889634);
  p.n_split = 1;
  return p;
}

}  // namespace

extern "C" {

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE_TOO_SMALL: return "FA_ERR_WORKSPACE_TOO_SMALL";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_version(void) { return "fa_gfx950 0.1"; }

int32_t fa_fwd_tile_rows(const fa_fwd_tuning* tuning) {
  FwdChoice c;
  if (pick_tuning(tuning, &c) != FA_OK) return 0;
  return c.splits > 1 ? fa::kFwdTileRows : fa::kFwdTileRows * c.qt;
}

fa_status fa_fwd_workspace_size(const fa_fwd_args* a, const fa_fwd_tuning* tuning, size_t* bytes) {
  if (bytes == nullptr) return FA_ERR_INVALID_ARGUMENT;
  Shape s;
  fa_status st = check_fwd(a, &s);
  if (st != FA_OK) return st;
  FwdChoice c;
  if ((st = pick_tuning(tuning, &c)) != FA_OK) return st;
  if ((st = check_variant(s, c)) != FA_OK) return st;
  const int splits = fwd_key_splits(s, c);
  *bytes = fwd_ws_layout(s, splits > 1 ? fa::kFwdTileRows : fa::kFwdTileRows * c.qt, splits).total;
  return FA_OK;
}

fa_status fa_fwd_build_schedule(const fa_fwd_args* a, const fa_fwd_tuning* tuning, void* workspace,
                                size_t workspace_bytes, void* stream) {
  Shape s;
  fa_status st = check_fwd(a, &s);
  if (st != FA_OK) return st;
  FwdChoice c;
  if ((st = pick_tuning(tuning, &c)) != FA_OK) return st;
  if ((st = check_variant(s, c)) != FA_OK) return st;
  if (!s.varlen) return FA_ERR_INVALID_ARGUMENT;
  const int tile_rows = fwd_key_splits(s, c) > 1 ? fa::kFwdTileRows : fa::kFwdTileRows * c.qt;
  const size_t need = fwd_ws_layout(s, tile_rows, 1).total;
  if (workspace == nullptr || workspace_bytes < need) return FA_ERR_WORKSPACE_TOO_SMALL;
  if ((uintptr_t)workspace % kAlign) return FA_ERR_INVALID_ARGUMENT;
  hipError_t e = fa::launch_fwd_schedule(s.cu_q, s.cu_k, s.batch, tile_rows, fa::kFwdBlockN, a->causal != 0,
                                         (int32_t*)workspace, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_exp2_probe(const float* x, float* y_poly, float* y_hw, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (x == nullptr || y_poly == nullptr || y_hw == nullptr))) return FA_ERR_INVALID_ARGUMENT;
  hipError_t e = fa::launch_exp2_probe(x, y_poly, y_hw, n, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd(const fa_fwd_args* a, const fa_fwd_tuning* tuning, void* workspace, size_t workspace_bytes,
                 void* stream) {
  Shape s;
  fa_status st = check_fwd(a, &s);
  if (st != FA_OK) return st;
  FwdChoice c;
  if ((st = pick_tuning(tuning, &c)) != FA_OK) return st;
  if ((st = check_variant(s, c)) != FA_OK) return st;
  const int splits = fwd_key_splits(s, c);
  if (splits > 1) c.qt = 1;  // the split path runs 128-row tiles
  const int tile_rows = fa::kFwdTileRows * c.qt;
  const FwdWs ws = fwd_ws_layout(s, tile_rows, splits);
  if (ws.total > 0 && (workspace == nullptr || workspace_bytes < ws.total)) return FA_ERR_WORKSPACE_TOO_SMALL;
  if (ws.total > 0 && (uintptr_t)workspace % kAlign) return FA_ERR_INVALID_ARGUMENT;
  if ((int64_t)fwd_max_items(s, tile_rows) * s.heads * splits > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (s.batch == 0 || s.total_q == 0) return FA_OK;

  fa::FwdParams p = make_fwd_params(a, s);
  p.n_qtiles = s.varlen ? 0 : (s.max_q + tile_rows - 1) / tile_rows;
  p.sched = (const int32_t*)workspace;
  if (splits > 1) {
    p.n_split = splits;
    p.part_lse = (float*)((char*)workspace + ws.lse_off);
    p.part_o = (float*)((char*)workspace + ws.o_off);
  }
  if (splits <= 1) {
    p.v16 = (uint16_t*)((char*)workspace + ws.v16_off);
    p.v_exp = (int32_t*)((char*)workspace + ws.vexp_off);
  }
  fa::FwdConfig cfg{s.d, c.qt, a->causal != 0, s.varlen, c.poly, c.tau, splits};
  hipStream_t strm = (hipStream_t)stream;
  if (s.varlen) {
    hipError_t e = fa::launch_fwd_schedule(s.cu_q, s.cu_k, s.batch, tile_rows, fa::kFwdBlockN, cfg.causal,
                                           (int32_t*)workspace, strm);
    if (e != hipSuccess) return FA_ERR_HIP;
  }
  if (splits <= 1 && s.total_k > 0 && fa::launch_fwd_vprep(p, s.d, s.varlen, strm) != hipSuccess) return FA_ERR_HIP;
  return fa::launch_fwd(p, cfg, strm) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---------------------------------------------------------------------------

namespace {

fa_status check_bwd(const fa_bwd_args* a, Shape* s) {
  if (a == nullptr) return FA_ERR_INVALID_ARGUMENT;
  fa_status st = check_shape(a->batch, a->seqlen_q, a->seqlen_k, a->num_heads, a->head_dim, a->cu_seqlens_q,
                             a->cu_seqlens_k, a->max_seqlen_q, a->max_seqlen_k, a->total_q, a->total_k, a->causal,
                             a->softmax_scale, s);
  if (st != FA_OK) return st;
  if (a->deterministic != 0 && a->deterministic != 1) return FA_ERR_INVALID_ARGUMENT;
  if (a->grad_dtype != FA_DTYPE_F32 && a->grad_dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARGUMENT;
  const int gb = a->grad_dtype == FA_DTYPE_F32 ? 4 : 2;
  if ((st = check_tensor(a->q, a->q_stride, *s, s->max_q, 2)) != FA_OK) return st;
  if ((st = check_tensor(a->k, a->k_stride, *s, s->max_k, 2)) != FA_OK) return st;
  if ((st = check_tensor(a->v, a->v_stride, *s, s->max_k, 2)) != FA_OK) return st;
  if ((st = check_tensor(a->o, a->o_stride, *s, s->max_q, 2)) != FA_OK) return st;
  if ((st = check_tensor(a->dout, a->do_stride, *s, s->max_q, 2)) != FA_OK) return st;
  if ((st = check_tensor(a->dq, a->dq_stride, *s, s->max_q, gb)) != FA_OK) return st;
  if ((st = check_tensor(a->dk, a->dk_stride, *s, s->max_k, gb)) != FA_OK) return st;
  if ((st = check_tensor(a->dv, a->dv_stride, *s, s->max_k, gb)) != FA_OK) return st;
  if (a->lse == nullptr || ((uintptr_t)a->lse & 3u)) return FA_ERR_INVALID_ARGUMENT;
  return FA_OK;
}

// Backward workspace: [fp32 dQ accumulator (atomic mode)] [row terms D_i] [work lists
// (variable length)] [maxima for the fp16 exponents] [Q16: H x total_q x D] [K16]
struct BwdLayout {
  size_t dq_acc, dvec, sched, stats, q16, k16, total;
};

BwdLayout bwd_layout(const Shape& s, bool deterministic) {
  BwdLayout l{};
  size_t off = 0;
  l.dq_acc = off;
  if (!deterministic) off += round_up(sizeof(float) * (size_t)s.total_q * s.heads * s.d);
  l.dvec = off;
  off += round_up(sizeof(float) * (size_t)s.total_q * s.heads);
  l.sched = off;
  if (s.varlen) {
    const size_t kv_items = (size_t)(s.total_k + fa::kBwdBlockN - 1) / fa::kBwdBlockN + s.batch;
    const size_t q_items = (size_t)(s.total_q + fa::kFwdTileRows - 1) / fa::kFwdTileRows + s.batch;
    off += round_up(sizeof(int32_t) * (1 + 2 * kv_items + 1 + 2 * q_items));
  }
  l.stats = off;
  off += round_up(4 * sizeof(uint32_t) * (1 + (size_t)fa::kBwdPreBlocks));
  l.q16 = off;
  off += round_up(sizeof(uint16_t) * (size_t)s.total_q * s.heads * s.d);
  l.k16 = off;
  off += round_up(sizeof(uint16_t) * (size_t)s.total_k * s.heads * s.d);
  l.total = off;
  return l;
}

// Scratch of the allocation-free backward (fa_bwd_noalloc): a file-scope device array,
// one copy per GPU, held until the process ends.  Host code never uses the array's
// name as an address (on the host it is only a stand-in for the symbol): each
// device's address is looked up once, with that device current, and kept here.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
__device__ __attribute__((aligned(256))) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's copy of `scratch`, or nullptr on a HIP error.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

fa_status fa_bwd_workspace_size(const fa_bwd_args* a, size_t* bytes) {
  if (bytes == nullptr) return FA_ERR_INVALID_ARGUMENT;
  Shape s;
  fa_status st = check_bwd(a, &s);
  if (st != FA_OK) return st;
  *bytes = bwd_layout(s, a->deterministic != 0).total;
  return FA_OK;
}

fa_status fa_bwd(const fa_bwd_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_phases(a, FA_BWD_PHASE_ALL, workspace, workspace_bytes, stream);
}

fa_status fa_bwd_noalloc(const fa_bwd_args* a, void* stream) {
  // every argument, and the workspace the request needs, is checked before any HIP call
  Shape s;
  fa_status st = check_bwd(a, &s);
  if (st != FA_OK) return st;
  if (bwd_layout(s, a->deterministic != 0).total > kNoallocScratchBytes) return FA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = device_scratch();
  if (ws == nullptr) return FA_ERR_HIP;
  return fa_bwd_phases(a, FA_BWD_PHASE_ALL, ws, kNoallocScratchBytes, stream);
}

size_t fa_bwd_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

fa_status fa_bwd_phases(const fa_bwd_args* a, int32_t phases, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (phases <= 0 || (phases & ~FA_BWD_PHASE_ALL)) return FA_ERR_INVALID_ARGUMENT;
  Shape s;
  fa_status st = check_bwd(a, &s);
  if (st != FA_OK) return st;
  const BwdLayout lay = bwd_layout(s, a->deterministic != 0);
  if (lay.total > 0 && (workspace == nullptr || workspace_bytes < lay.total)) return FA_ERR_WORKSPACE_TOO_SMALL;
  if (lay.total > 0 && (uintptr_t)workspace % kAlign) return FA_ERR_INVALID_ARGUMENT;
  // Empty problems: nothing to write.  (Queries without keys get dQ = 0 and keys
  // without queries get dK = dV = 0 from the kernels themselves.)
  if (s.batch == 0 || (s.total_q == 0 && s.total_k == 0)) return FA_OK;
  fa::BwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.dout = a->dout; p.lse = a->lse;
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  p.q_sb = a->q_stride[0]; p.q_ss = a->q_stride[1]; p.q_sh = a->q_stride[2];
  p.k_sb = a->k_stride[0]; p.k_ss = a->k_stride[1]; p.k_sh = a->k_stride[2];
  p.v_sb = a->v_stride[0]; p.v_ss = a->v_stride[1]; p.v_sh = a->v_stride[2];
  p.o_sb = a->o_stride[0]; p.o_ss = a->o_stride[1]; p.o_sh = a->o_stride[2];
  p.do_sb = a->do_stride[0]; p.do_ss = a->do_stride[1]; p.do_sh = a->do_stride[2];
  p.dq_sb = a->dq_stride[0]; p.dq_ss = a->dq_stride[1]; p.dq_sh = a->dq_stride[2];
  p.dk_sb = a->dk_stride[0]; p.dk_ss = a->dk_stride[1]; p.dk_sh = a->dk_stride[2];
  p.dv_sb = a->dv_stride[0]; p.dv_ss = a->dv_stride[1]; p.dv_sh = a->dv_stride[2];
  p.batch = s.batch;
  p.seqlen_q = s.max_q;
  p.seqlen_k = s.max_k;
  p.heads = s.heads;
  p.cu_q = s.cu_q;
  p.cu_k = s.cu_k;
  p.total_q = s.total_q;
  p.total_k = s.total_k;
  p.max_seqlen_q = s.max_q;
  p.max_seqlen_k = s.max_k;
  p.scale = a->softmax_scale;
  p.scale_log2 = (float)((double)a->softmax_scale * 1.4426950408889634);
  p.causal = a->causal != 0;
  p.varlen = s.varlen;
  p.deterministic = a->deterministic != 0;
  p.grad_bf16 = a->grad_dtype == FA_DTYPE_BF16;
  p.head_dim = s.d;
  char* ws = (char*)workspace;
  p.dq_acc = a->deterministic ? nullptr : (float*)(ws + lay.dq_acc);
  p.dvec = (float*)(ws + lay.dvec);
  p.sched = s.varlen ? (int32_t*)(ws + lay.sched) : nullptr;
  p.stats = (uint32_t*)(ws + lay.stats);
  p.q16 = (uint16_t*)(ws + lay.q16);
  p.k16 = (uint16_t*)(ws + lay.k16);
  return fa::launch_bwd(p, phases, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
