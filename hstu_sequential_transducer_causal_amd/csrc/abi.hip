// abi.hip -- the C ABI of libhstu.so (declared in include/hstu.h): argument
// validation, workspace carving and kernel dispatch on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "internal.h"
#include "../../include/hstu.h"

namespace hstu {

int device_cu_count() {
    static int counts[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (counts[dev] == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        counts[dev] = c;
    }
    return counts[dev];
}

}  // namespace hstu

namespace {

thread_local char g_last_error[512] = "";

hstu_status fail(hstu_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

hstu_status ok() {
    g_last_error[0] = '\0';
    return HSTU_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int tile_m_for(int dtype) { return dtype == HSTU_BF16 ? hstu::kBf16TileM : hstu::kF32TileM; }
int tile_n_for(int dtype) { return dtype == HSTU_BF16 ? hstu::kBf16TileN : hstu::kF32TileN; }

// Checks everything that can be checked on the host; with need_epi the
// LN*U epilogue arguments are required even if y is NULL.
hstu_status validate_attn(const hstu_attn_args* a, bool need_epi) {
    if (!a) return fail(HSTU_ERR_ARG, "args is NULL");
    if (a->struct_size != sizeof(hstu_attn_args))
        return fail(HSTU_ERR_ARG, "struct_size %u != sizeof(hstu_attn_args) %zu", a->struct_size,
                    sizeof(hstu_attn_args));
    if (a->B < 0) return fail(HSTU_ERR_ARG, "B = %d < 0", a->B);
    if (a->H < 1) return fail(HSTU_ERR_ARG, "H = %d < 1", a->H);
    if (a->d_qk < 1 || a->d_v < 1) return fail(HSTU_ERR_ARG, "head dims must be >= 1");
    if (a->max_seq_len < 0 || a->max_seq_len > hstu::kMaxSeqLen)
        return fail(HSTU_ERR_ARG, "max_seq_len %d outside [0, %d]", a->max_seq_len, hstu::kMaxSeqLen);
    if (a->num_rows < 0) return fail(HSTU_ERR_ARG, "num_rows < 0");
    if (a->dtype != HSTU_F32 && a->dtype != HSTU_BF16) return fail(HSTU_ERR_ARG, "unknown dtype %d", a->dtype);
    if (a->act != HSTU_ACT_SILU && a->act != HSTU_ACT_IDENTITY) return fail(HSTU_ERR_ARG, "unknown act %d", a->act);
    if (a->dtype == HSTU_BF16 && !(a->d_qk == 128 && a->d_v == 128))
        return fail(HSTU_ERR_UNSUPPORTED, "bf16 needs d_qk = d_v = 128 (got %d, %d)", a->d_qk, a->d_v);
    if (a->dtype == HSTU_F32 && !(a->d_qk == a->d_v && (a->d_qk == 32 || a->d_qk == 64)))
        return fail(HSTU_ERR_UNSUPPORTED, "fp32 needs d_qk = d_v in {32, 64} (got %d, %d)", a->d_qk, a->d_v);
    if (a->num_pos_buckets < 1 || a->num_pos_buckets > hstu::kMaxPosBuckets)
        return fail(HSTU_ERR_ARG, "num_pos_buckets %d outside [1, %d]", a->num_pos_buckets, hstu::kMaxPosBuckets);
    if (a->num_time_buckets < 1) return fail(HSTU_ERR_ARG, "num_time_buckets %d < 1", a->num_time_buckets);
    if (a->rab_pos_head_stride < 0 || a->rab_time_head_stride < 0)
        return fail(HSTU_ERR_ARG, "negative bias-table head stride");
    if (!std::isfinite(a->alpha)) return fail(HSTU_ERR_ARG, "alpha is not finite");
    const int64_t hq = int64_t(a->H) * a->d_qk, hv = int64_t(a->H) * a->d_v;
    if (a->q_stride < hq || a->k_stride < hq) return fail(HSTU_ERR_ARG, "q/k stride < H*d_qk");
    if (a->v_stride < hv || a->o_stride < hv) return fail(HSTU_ERR_ARG, "v/o stride < H*d_v");
    const bool epi = need_epi || a->y != nullptr;
    if (epi) {
        if (!(a->ln_eps > 0.0f) || !std::isfinite(a->ln_eps)) return fail(HSTU_ERR_ARG, "ln_eps must be > 0");
        if (a->u_stride < hv) return fail(HSTU_ERR_ARG, "u stride < H*d_v");
        if (a->y && a->y_stride < hv) return fail(HSTU_ERR_ARG, "y stride < H*d_v");
        if (hv % 8 != 0 || hv > 4096) return fail(HSTU_ERR_UNSUPPORTED, "epilogue needs H*d_v %% 8 == 0 and <= 4096");
    }
    if (a->B > 0) {
        if (!a->seq_offsets) return fail(HSTU_ERR_ARG, "seq_offsets is NULL");
        if (!a->q || !a->k || !a->v || !a->o) return fail(HSTU_ERR_ARG, "q, k, v and o must be non-NULL");
        if (!a->timestamps) return fail(HSTU_ERR_ARG, "timestamps is NULL");
        if (!a->rab_pos || !a->rab_time) return fail(HSTU_ERR_ARG, "bias tables must be non-NULL");
        if (epi && !a->u) return fail(HSTU_ERR_ARG, "u is NULL but the LN*U epilogue is requested");
        if (a->dtype == HSTU_BF16) {
            const int64_t row_bytes = 2 * (a->k_stride > a->v_stride ? a->k_stride : a->v_stride);
            if (int64_t(a->max_seq_len) * row_bytes > int64_t(0x7fffffff))
                return fail(HSTU_ERR_UNSUPPORTED, "max_seq_len * K/V row bytes must stay below 2^31");
            if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || (a->q_stride % 8) || (a->k_stride % 8) ||
                (a->v_stride % 8))
                return fail(HSTU_ERR_UNSUPPORTED, "bf16 q/k/v rows must be 16-byte aligned");
        }
        if (epi) {
            const int64_t vec = a->dtype == HSTU_BF16 ? 8 : 4;
            if (!aligned16(a->o) || (a->o_stride % vec) || !aligned16(a->u) || (a->u_stride % vec) ||
                (a->y && (!aligned16(a->y) || (a->y_stride % vec))))
                return fail(HSTU_ERR_UNSUPPORTED, "epilogue rows must be 16-byte aligned");
        }
    }
    return HSTU_OK;
}

hstu_status check_workspace(void* ws, size_t have, size_t need) {
    if (need == 0) return HSTU_OK;
    if (!ws) return fail(HSTU_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned16(ws)) return fail(HSTU_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    if (have < need) return fail(HSTU_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", have, need);
    return HSTU_OK;
}

hstu_status device_error(hipError_t e, const char* what) {
    return fail(HSTU_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// The batch structure on the device (offsets, lengths, candidate counts),
// checked by one small kernel: hstu_validate_offsets, and every call when the
// environment sets HSTU_VALIDATE=1 (a synchronising debug aid).
hstu_status device_check_batch(int B, int64_t num_rows, int max_seq_len, const int32_t* offsets,
                               const int32_t* lengths, const int32_t* ncand, hipStream_t stream,
                               bool packed = false) {
    hstu::ValidateArgs v;
    v.packed = packed ? 1 : 0;
    v.B = B;
    v.num_rows = num_rows;
    v.max_seq_len = max_seq_len;
    v.offsets = offsets;
    v.lengths = lengths;
    v.ncand = ncand;
    int64_t first = -1;
    const hipError_t e = hstu::validate_batch(v, stream, &first);
    if (e != hipSuccess) return device_error(e, "batch validation");
    if (first < 0) return ok();
    static const char* const what[8] = {"", "offsets[0] < 0", "offsets decrease", "offsets[B] > num_rows",
                                        "seq_lengths[b] outside [0, offsets[b+1] - offsets[b]]",
                                        "length > max_seq_len", "num_candidates[b] outside [0, length]",
                                        "a layer needs packed offsets (offsets[0] = 0, offsets[B] = num_rows)"};
    return fail(HSTU_ERR_ARG, "sequence %lld: %s", (long long)(first / 8), what[first % 8]);
}

bool validate_env() {
    const char* v = std::getenv("HSTU_VALIDATE");
    return v && v[0] == '1' && v[1] == '\0';
}

hstu_status maybe_check_batch(const hstu_attn_args* a, hipStream_t stream) {
    if (!validate_env()) return HSTU_OK;
    return device_check_batch(a->B, a->num_rows, a->max_seq_len, a->seq_offsets, a->seq_lengths,
                              a->num_candidates, stream);
}

struct Sched {
    hstu::SchedLayout layout;
    int32_t* ctrl;
    int32_t* qscan;
    hstu::WorkItem* items;
    hstu::ItemSeq* item_seq;
    hstu::SplitBlock* split;
    float* partial;
    uint32_t* stats;
    uint32_t* enc;
    int32_t* rowmap;   // NULL unless row blocks may be split
};

// The fp32 core needs neither row codes nor block ranges, and never splits.
hstu::SchedLayout sched_layout_for(const hstu_attn_args* a, size_t base) {
    const bool bf16 = a->dtype == HSTU_BF16;
    return hstu::sched_layout(a->B, a->H, a->max_seq_len, tile_m_for(a->dtype), bf16 ? a->d_v : 0,
                              bf16 ? a->num_rows : 0, base);
}

// The same layout with at most max_slots split-partial slots.
hstu::SchedLayout sched_layout_for_slots(const hstu_attn_args* a, int max_slots, size_t base = 0) {
    const bool bf16 = a->dtype == HSTU_BF16;
    return hstu::sched_layout(a->B, a->H, a->max_seq_len, tile_m_for(a->dtype), bf16 ? a->d_v : 0,
                              bf16 ? a->num_rows : 0, base, max_slots);
}

Sched carve_sched(const hstu_attn_args* a, void* ws, size_t base, int max_slots = hstu::kMaxPartialSlots) {
    Sched s;
    s.layout = sched_layout_for_slots(a, max_slots, base);
    uint8_t* w = static_cast<uint8_t*>(ws);
    s.ctrl = reinterpret_cast<int32_t*>(w + s.layout.off_ctrl);
    s.qscan = reinterpret_cast<int32_t*>(w + s.layout.off_qscan);
    s.items = reinterpret_cast<hstu::WorkItem*>(w + s.layout.off_items);
    s.item_seq = reinterpret_cast<hstu::ItemSeq*>(w + s.layout.off_item_seq);
    s.split = reinterpret_cast<hstu::SplitBlock*>(w + s.layout.off_split);
    s.partial = reinterpret_cast<float*>(w + s.layout.off_part);
    s.stats = reinterpret_cast<uint32_t*>(w + s.layout.off_stats);
    s.enc = reinterpret_cast<uint32_t*>(w + s.layout.off_enc);
    s.rowmap = s.layout.part_slots > 0 ? reinterpret_cast<int32_t*>(w + s.layout.off_rowmap) : nullptr;
    return s;
}

hstu::SchedArgs make_sched_args(const hstu_attn_args* a, const Sched& s, bool cand_only) {
    hstu::SchedArgs sa;
    sa.cand_only = cand_only ? 1 : 0;
    sa.kv_mode = 0;
    sa.B = a->B;
    sa.max_seq_len = a->max_seq_len;
    sa.cap = (int64_t)s.layout.cap;
    sa.cap_pieces = (int64_t)s.layout.cap_pieces;
    sa.H = a->H;
    sa.slots = a->dtype == HSTU_BF16 ? hstu::attn_bf16_slots() : 0;
    sa.part_slots = s.layout.part_slots;
    sa.split = s.split;
    sa.offsets = a->seq_offsets;
    sa.lengths = a->seq_lengths;
    sa.ncand = a->num_candidates;
    sa.tile_m = tile_m_for(a->dtype);
    sa.tile_n = tile_n_for(a->dtype);
    sa.ctrl = s.ctrl;
    sa.qscan = s.qscan;
    sa.items = s.items;
    sa.item_seq = s.item_seq;
    const bool bf16 = a->dtype == HSTU_BF16;
    sa.ts = a->timestamps;
    sa.enc = bf16 ? s.enc : nullptr;
    sa.stats = s.stats;
    sa.nblk = s.layout.nblk;
    sa.cap_blk = bf16 ? (int64_t)s.layout.cap_blk : 0;
    return sa;
}

hipError_t run_sched(const hstu_attn_args* a, const Sched& s, hipStream_t stream, bool cand_only = false) {
    return hstu::launch_sched(make_sched_args(a, s, cand_only), stream);
}

hipError_t run_core(const hstu_attn_args* a, const Sched& s, hipStream_t stream) {
    hstu::AttnCoreArgs c;
    c.H = a->H;
    c.d = a->d_qk;
    c.offsets = a->seq_offsets;
    c.lengths = a->seq_lengths;
    c.ncand = a->num_candidates;
    c.q = a->q; c.q_stride = a->q_stride;
    c.k = a->k; c.k_stride = a->k_stride;
    c.v = a->v; c.v_stride = a->v_stride;
    c.ts = a->timestamps;
    c.rab_pos = a->rab_pos; c.P = a->num_pos_buckets; c.rp_head_stride = a->rab_pos_head_stride;
    c.rab_time = a->rab_time; c.NT = a->num_time_buckets; c.rt_head_stride = a->rab_time_head_stride;
    c.alpha = a->alpha;
    c.act = a->act;
    c.o = a->o; c.o_stride = a->o_stride;
    c.items = s.items;
    c.item_seq = s.item_seq;
    c.ctrl = s.ctrl;
    c.cursor = s.ctrl + 1;
    c.partial = s.partial;
    c.rowmap = s.rowmap;
    c.nblk = s.layout.nblk;
    c.stats = s.stats;
    c.enc = s.enc;
    c.num_rows = a->num_rows;
    // the events travel with the launch itself (no marker packets around it)
    c.ev_begin = static_cast<hipEvent_t>(a->ev_core_begin);
    c.ev_end = static_cast<hipEvent_t>(a->ev_core_end);
    return a->dtype == HSTU_BF16 ? hstu::launch_attn_bf16(c, stream) : hstu::launch_attn_f32(c, stream);
}

// Adds up the partial sums of split row blocks into O (bf16 core only).
hipError_t run_combine(const hstu_attn_args* a, const Sched& s, hipStream_t stream) {
    if (a->dtype != HSTU_BF16 || s.layout.part_slots <= 0 || a->H <= 0) return hipSuccess;
    hstu::CombineArgs c;
    c.H = a->H;
    c.d = a->d_v;
    c.BM = hstu::kBf16TileM;
    c.offsets = a->seq_offsets;
    c.lengths = a->seq_lengths;
    c.ctrl = s.ctrl;
    c.split = s.split;
    c.partial = s.partial;
    c.o = a->o; c.o_stride = a->o_stride;
    // a split block takes at least two slots per head
    c.max_blocks = std::min<int64_t>((int64_t)s.layout.cap, s.layout.part_slots / (2 * a->H));
    return hstu::launch_combine(c, stream);
}

hipError_t run_ln_gate(const hstu_attn_args* a, const Sched& s, const float* w, float* scores,
                       int score_stride, bool cand_only, hipStream_t stream) {
    hstu::LnGateArgs l;
    l.B = a->B;
    l.num_rows = a->num_rows;
    l.width = a->H * a->d_v;
    l.dtype = a->dtype;
    l.offsets = a->seq_offsets;
    l.lengths = a->seq_lengths;
    l.ncand = a->num_candidates;
    l.o = a->o; l.o_stride = a->o_stride;
    l.u = a->u; l.u_stride = a->u_stride;
    l.y = a->y; l.y_stride = a->y_stride;
    l.eps = a->ln_eps;
    l.w = w;
    l.scores = scores;
    l.score_stride = score_stride;
    // split row blocks are added up here (no separate combine pass)
    l.rowmap = s.rowmap;
    l.partial = s.partial;
    l.H = a->H;
    l.d = a->d_v;
    l.BM = hstu::kBf16TileM;
    l.cand_only = cand_only ? 1 : 0;
    l.ev_begin = static_cast<hipEvent_t>(a->ev_epi_begin);
    l.ev_end = static_cast<hipEvent_t>(a->ev_epi_end);
    return hstu::launch_ln_gate(l, stream);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---- the scratch buffer of hstu_attn_fwd_noalloc
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid it): a file-scope
// device array that every GPU the library runs on holds from module load to
// the end of the process.  Host code must not pass the array's name to a
// kernel (on the host it is only a stand-in, not the device address): its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept.  Calls on one GPU share the array (and
// leave their contents in it); the scheduler kernel rewrites every word a
// call reads before the call reads it, including the work cursors, so
// nothing needs clearing -- but calls that may overlap on one GPU (streams
// without ordering between them) race.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// ---- M-FALCON against a history cache

hstu_status validate_cached(const hstu_mfalcon_cached_args* m) {
    if (!m) return fail(HSTU_ERR_ARG, "args is NULL");
    if (m->struct_size != sizeof(hstu_mfalcon_cached_args))
        return fail(HSTU_ERR_ARG, "struct_size %u != sizeof(hstu_mfalcon_cached_args) %zu", m->struct_size,
                    sizeof(hstu_mfalcon_cached_args));
    if (m->B < 0 || m->H < 1) return fail(HSTU_ERR_ARG, "B >= 0 and H >= 1 required");
    if (m->d != 128) return fail(HSTU_ERR_UNSUPPORTED, "d must be 128 (got %d)", m->d);
    if (m->max_hist_len < 0 || m->max_hist_len > hstu::kMaxSeqLen || m->max_cands < 0 ||
        m->max_cands > hstu::kMaxSeqLen)
        return fail(HSTU_ERR_ARG, "max_hist_len and max_cands must lie in [0, %d]", hstu::kMaxSeqLen);
    if (m->num_hist_rows < 0 || m->num_cand_rows < 0) return fail(HSTU_ERR_ARG, "row counts must be >= 0");
    if (m->num_pos_buckets < 1 || m->num_pos_buckets > hstu::kMaxPosBuckets)
        return fail(HSTU_ERR_ARG, "num_pos_buckets outside [1, %d]", hstu::kMaxPosBuckets);
    if (m->num_time_buckets < 1) return fail(HSTU_ERR_ARG, "num_time_buckets < 1");
    if (m->rab_pos_head_stride < 0 || m->rab_time_head_stride < 0) return fail(HSTU_ERR_ARG, "negative head stride");
    if (!std::isfinite(m->alpha)) return fail(HSTU_ERR_ARG, "alpha is not finite");
    if (!(m->ln_eps > 0.0f) || !std::isfinite(m->ln_eps)) return fail(HSTU_ERR_ARG, "ln_eps must be > 0");
    if (m->score_stride < std::max(1, m->max_cands)) return fail(HSTU_ERR_ARG, "score_stride < max_cands");
    const int64_t hd = int64_t(m->H) * m->d;
    if (hd > 4096) return fail(HSTU_ERR_UNSUPPORTED, "H*d must be <= 4096");
    const int64_t strides[7] = {m->k_hist_stride, m->v_hist_stride, m->q_stride, m->k_stride, m->v_stride,
                                m->u_stride, m->o ? m->o_stride : hd};
    for (int64_t st : strides)
        if (st < hd || st % 8) return fail(HSTU_ERR_ARG, "row strides must be >= H*d and multiples of 8");
    if (int64_t(m->max_hist_len) * 2 * std::max(m->k_hist_stride, m->v_hist_stride) > int64_t(0x7fffffff))
        return fail(HSTU_ERR_UNSUPPORTED, "max_hist_len * K/V row bytes must stay below 2^31");
    if (m->B > 0) {
        if (!m->hist_offsets || !m->cand_offsets || !m->k_hist || !m->v_hist || !m->ts_hist || !m->q || !m->k ||
            !m->v || !m->u || !m->ts_cand || !m->rab_pos || !m->rab_time || !m->w || !m->scores)
            return fail(HSTU_ERR_ARG, "a required pointer is NULL");
        const void* ptrs[7] = {m->k_hist, m->v_hist, m->q, m->k, m->v, m->u, m->o ? m->o : m->q};
        for (const void* ptr : ptrs)
            if (!aligned16(ptr)) return fail(HSTU_ERR_UNSUPPORTED, "bf16 rows must be 16-byte aligned");
    }
    return HSTU_OK;
}

struct CachedWs {
    hstu::SchedLayout cand;      // candidates' work list, codes, split slots, row map
    size_t kstats, kenc, o, total;
    int nblk_k;
};

CachedWs cached_ws(const hstu_mfalcon_cached_args* m) {
    CachedWs w;
    w.cand = hstu::sched_layout(m->B, m->H, m->max_cands, hstu::kBf16TileM, m->d, m->num_cand_rows, 0);
    w.nblk_k = (m->max_hist_len + hstu::kTsBlock - 1) / hstu::kTsBlock;
    w.kstats = align256(w.cand.bytes);
    w.kenc = align256(w.kstats + size_t(m->B) * w.nblk_k * 2 * sizeof(uint32_t));
    w.o = align256(w.kenc + size_t(m->num_hist_rows) * sizeof(uint32_t));
    w.total = align256(w.o + (m->o ? 0 : size_t(m->num_cand_rows) * m->H * m->d * 2));
    return w;
}

// ---- gradients

hstu_status validate_bwd(const hstu_attn_bwd_args* g) {
    if (!g) return fail(HSTU_ERR_ARG, "args is NULL");
    if (g->struct_size != sizeof(hstu_attn_bwd_args))
        return fail(HSTU_ERR_ARG, "struct_size %u != sizeof(hstu_attn_bwd_args) %zu", g->struct_size,
                    sizeof(hstu_attn_bwd_args));
    const bool with_dy = g->dy != nullptr;
    hstu_attn_args a = g->attn;
    a.y = nullptr;
    if (!with_dy && a.o == nullptr) {   // O is read only to differentiate the gate
        a.o = const_cast<void*>(a.v);
        a.o_stride = a.v_stride;
    }
    hstu_status st = validate_attn(&a, with_dy);
    if (st != HSTU_OK) return st;
    if (a.dtype != HSTU_BF16) return fail(HSTU_ERR_UNSUPPORTED, "gradients need bf16 inputs (d = 128)");
    if (!hstu::attn_bwd_tables_fit(a.num_pos_buckets, a.num_time_buckets))
        return fail(HSTU_ERR_UNSUPPORTED, "gradients support num_pos_buckets up to about 5200");
    const int64_t hd = int64_t(a.H) * a.d_v;
    if (g->dq_stride < hd || g->dk_stride < hd || g->dv_stride < hd)
        return fail(HSTU_ERR_ARG, "dq/dk/dv stride < H*d");
    if (with_dy && (g->dy_stride < hd || (g->du && g->du_stride < hd)))
        return fail(HSTU_ERR_ARG, "dy/du stride < H*d");
    if (!with_dy && g->dout_stride < hd) return fail(HSTU_ERR_ARG, "dout stride < H*d");
    if (a.B > 0) {
        if (!g->dq || !g->dk || !g->dv) return fail(HSTU_ERR_ARG, "dq, dk and dv must be non-NULL");
        if (!with_dy && !g->dout) return fail(HSTU_ERR_ARG, "one of dy and dout is required");
        auto rows_ok = [](const void* p, int64_t stride) { return aligned16(p) && stride % 8 == 0; };
        if (!rows_ok(g->dq, g->dq_stride) || !rows_ok(g->dk, g->dk_stride) || !rows_ok(g->dv, g->dv_stride) ||
            (with_dy && !rows_ok(g->dy, g->dy_stride)) || (g->du && !rows_ok(g->du, g->du_stride)) ||
            (!with_dy && !rows_ok(g->dout, g->dout_stride)))
            return fail(HSTU_ERR_UNSUPPORTED, "gradient rows must be 16-byte aligned");
        const int64_t gstride = with_dy ? hd : g->dout_stride;
        const int64_t widest = std::max(a.q_stride, gstride);
        if (int64_t(a.max_seq_len) * 2 * widest > int64_t(0x7fffffff))
            return fail(HSTU_ERR_UNSUPPORTED, "max_seq_len * Q/dO row bytes must stay below 2^31");
        // one 32-row query tile's G blocks (fp32, every head) in one buffer range
        if ((int64_t(a.max_seq_len) / 32 + 1) * a.H * 4096 > int64_t(0x7fffffff))
            return fail(HSTU_ERR_UNSUPPORTED, "(max_seq_len / 32 + 1) * H * 4096 must stay below 2^31");
    }
    return HSTU_OK;
}

struct BwdWs {
    hstu::SchedLayout q, kv;   // query-major and key-major work lists
    size_t dout, part, part2, gbase, gbuf, kp, total;
    int64_t gcap;              // G blocks (32 x 32 fp32, per head) the buffer holds
};

BwdWs bwd_ws(const hstu_attn_bwd_args* g) {
    const hstu_attn_args& a = g->attn;
    BwdWs w;
    w.q = hstu::sched_layout(a.B, a.H, a.max_seq_len, hstu::kBf16TileM, 0, a.num_rows, 0);
    w.kv = hstu::sched_layout(a.B, a.H, a.max_seq_len, hstu::kBf16TileM, 0, 0, w.q.bytes);
    w.dout = align256(w.kv.bytes);
    w.part = align256(w.dout + (g->dy ? size_t(a.num_rows) * size_t(a.H) * size_t(a.d_v) * 2 : 0));
    w.part2 = align256(w.part + sizeof(float) * hstu::attn_bwd_rab_part_floats(
                                                    (int64_t)w.q.cap, a.H, a.num_pos_buckets, a.num_time_buckets));
    w.gbase = align256(w.part2 + sizeof(float) * hstu::attn_bwd_rab_part2_floats(a.H, a.num_pos_buckets,
                                                                                  a.num_time_buckets));
    w.gbuf = align256(w.gbase + sizeof(int64_t) * size_t(a.B > 0 ? a.B : 0));
    w.gcap = hstu::attn_bwd_g_blocks(a.B, a.max_seq_len, a.num_rows);
    w.kp = align256(w.gbuf + size_t(w.gcap) * size_t(a.H) * 1024 * sizeof(float));
    w.total = align256(w.kp + size_t(a.B > 0 ? a.B : 0) * size_t(w.q.nblk) * size_t(a.H) * 8192);
    return w;
}

Sched carve_layout(const hstu::SchedLayout& l, void* ws) {
    Sched s;
    s.layout = l;
    uint8_t* w = static_cast<uint8_t*>(ws);
    s.ctrl = reinterpret_cast<int32_t*>(w + l.off_ctrl);
    s.qscan = reinterpret_cast<int32_t*>(w + l.off_qscan);
    s.items = reinterpret_cast<hstu::WorkItem*>(w + l.off_items);
    s.item_seq = reinterpret_cast<hstu::ItemSeq*>(w + l.off_item_seq);
    s.split = reinterpret_cast<hstu::SplitBlock*>(w + l.off_split);
    s.partial = nullptr;
    s.stats = reinterpret_cast<uint32_t*>(w + l.off_stats);
    s.enc = reinterpret_cast<uint32_t*>(w + l.off_enc);
    s.rowmap = nullptr;
    return s;
}

}  // namespace

extern "C" {

int hstu_abi_version(void) { return HSTU_ABI_VERSION; }

const char* hstu_status_string(hstu_status s) {
    switch (s) {
        case HSTU_OK: return "HSTU_OK";
        case HSTU_ERR_ARG: return "HSTU_ERR_ARG: invalid argument";
        case HSTU_ERR_UNSUPPORTED: return "HSTU_ERR_UNSUPPORTED: no kernel for this shape or dtype";
        case HSTU_ERR_WORKSPACE: return "HSTU_ERR_WORKSPACE: workspace missing or too small";
        case HSTU_ERR_DEVICE: return "HSTU_ERR_DEVICE: HIP call or kernel launch failed";
        default: return "unknown hstu_status";
    }
}

const char* hstu_last_error(void) { return g_last_error; }

size_t hstu_attn_workspace_bytes(const hstu_attn_args* a) {
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    hstu_status st = validate_attn(a, false);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != HSTU_OK) return 0;
    return sched_layout_for(a, 0).bytes;
}

hstu_status hstu_attn_fwd(const hstu_attn_args* a, void* ws, size_t ws_bytes, void* stream_) {
    hstu_status st = validate_attn(a, false);
    if (st != HSTU_OK) return st;
    if (a->B == 0) return ok();
    st = maybe_check_batch(a, static_cast<hipStream_t>(stream_));
    if (st != HSTU_OK) return st;
    const size_t need = sched_layout_for(a, 0).bytes;
    st = check_workspace(ws, ws_bytes, need);
    if (st != HSTU_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    Sched s = carve_sched(a, ws, 0);
    hipError_t e = run_sched(a, s, stream);
    if (e != hipSuccess) return device_error(e, "scheduler launch");
    e = run_core(a, s, stream);
    if (e != hipSuccess) return device_error(e, "attention launch");
    if (a->y) {
        e = run_ln_gate(a, s, nullptr, nullptr, 0, false, stream);
        if (e != hipSuccess) return device_error(e, "epilogue launch");
    } else {
        e = run_combine(a, s, stream);
        if (e != hipSuccess) return device_error(e, "split combine launch");
    }
    return ok();
}

size_t hstu_attn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

hstu_status hstu_attn_fwd_noalloc(const hstu_attn_args* a, void* stream_) {
    hstu_status st = validate_attn(a, false);
    if (st != HSTU_OK) return st;
    if (a->B == 0) return ok();
    // the layout hstu_attn_fwd would use, with as many split-partial slots
    // as still fit (each holds BM x d_v fp32): the size check is host
    // arithmetic, done before any HIP call
    hstu::SchedLayout l = sched_layout_for(a, 0);
    if (l.bytes > kNoAllocScratchBytes && l.part_slots > 0) {
        const size_t slot_bytes = size_t(hstu::kBf16TileM) * size_t(a->d_v) * sizeof(float);
        const size_t fixed = sched_layout_for_slots(a, 0).bytes;
        const int fit = fixed >= kNoAllocScratchBytes ? 0 : (int)((kNoAllocScratchBytes - fixed) / slot_bytes);
        // the item list grows with the slots as well: step down until it fits
        int slots = std::min(fit, l.part_slots);
        for (;;) {
            l = sched_layout_for_slots(a, slots);
            if (l.bytes <= kNoAllocScratchBytes || slots == 0) break;
            slots = slots * 7 / 8;
        }
    }
    if (l.bytes > kNoAllocScratchBytes)
        return fail(HSTU_ERR_WORKSPACE,
                    "hstu_attn_fwd_noalloc: the call needs %zu bytes of scratch, more than the %zu the library holds "
                    "per GPU (use hstu_attn_fwd with a workspace)",
                    l.bytes, kNoAllocScratchBytes);
    void* ws = nullptr;
    hipError_t e = noalloc_scratch(&ws);
    if (e != hipSuccess) return device_error(e, "locating the library's scratch buffer");
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    Sched s = carve_sched(a, ws, 0, l.part_slots);
    e = run_sched(a, s, stream);
    if (e != hipSuccess) return device_error(e, "scheduler launch");
    e = run_core(a, s, stream);
    if (e != hipSuccess) return device_error(e, "attention launch");
    if (a->y) {
        e = run_ln_gate(a, s, nullptr, nullptr, 0, false, stream);
        if (e != hipSuccess) return device_error(e, "epilogue launch");
    } else {
        e = run_combine(a, s, stream);
        if (e != hipSuccess) return device_error(e, "split combine launch");
    }
    return ok();
}

size_t hstu_mfalcon_workspace_bytes(const hstu_mfalcon_args* m) {
    if (!m || m->struct_size != sizeof(hstu_mfalcon_args)) return 0;
    return hstu_attn_workspace_bytes(&m->attn);
}

hstu_status mfalcon_score(const hstu_mfalcon_args* m, void* ws, size_t ws_bytes, void* stream_) {
    if (!m) return fail(HSTU_ERR_ARG, "args is NULL");
    if (m->struct_size != sizeof(hstu_mfalcon_args))
        return fail(HSTU_ERR_ARG, "struct_size %u != sizeof(hstu_mfalcon_args) %zu", m->struct_size,
                    sizeof(hstu_mfalcon_args));
    const hstu_attn_args* a = &m->attn;
    hstu_status st = validate_attn(a, true);
    if (st != HSTU_OK) return st;
    if (m->score_stride < 1) return fail(HSTU_ERR_ARG, "score_stride < 1");
    if (a->B == 0) return ok();
    st = maybe_check_batch(a, static_cast<hipStream_t>(stream_));
    if (st != HSTU_OK) return st;
    if (!a->num_candidates) return fail(HSTU_ERR_ARG, "num_candidates is required for M-FALCON");
    if (!m->w || !m->scores) return fail(HSTU_ERR_ARG, "w and scores must be non-NULL");
    if (m->candidates_only && a->y)
        return fail(HSTU_ERR_ARG, "candidates_only leaves history rows of O unwritten: attn.y must be NULL");
    const size_t need = sched_layout_for(a, 0).bytes;
    st = check_workspace(ws, ws_bytes, need);
    if (st != HSTU_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    Sched s = carve_sched(a, ws, 0);
    hipError_t e = run_sched(a, s, stream, m->candidates_only != 0);
    if (e != hipSuccess) return device_error(e, "scheduler launch");
    e = run_core(a, s, stream);
    if (e != hipSuccess) return device_error(e, "attention launch");
    e = run_ln_gate(a, s, m->w, m->scores, m->score_stride, m->candidates_only != 0, stream);
    if (e != hipSuccess) return device_error(e, "epilogue launch");
    return ok();
}

}  // extern "C"

namespace {

hstu_status validate_layer(const hstu_layer_args* l, bool f2 = true) {
    if (!l) return fail(HSTU_ERR_ARG, "args is NULL");
    if (l->struct_size != sizeof(hstu_layer_args))
        return fail(HSTU_ERR_ARG, "struct_size %u != sizeof(hstu_layer_args) %zu", l->struct_size,
                    sizeof(hstu_layer_args));
    if (l->B < 0 || l->H < 1 || l->D < 1) return fail(HSTU_ERR_ARG, "B >= 0, H >= 1, D >= 1 required");
    if (l->d != 128) return fail(HSTU_ERR_UNSUPPORTED, "layer needs d = 128 (got %d)", l->d);
    if (l->D % 128 != 0 || (4 * l->H * l->d) % 128 != 0)
        return fail(HSTU_ERR_UNSUPPORTED, "layer needs D %% 128 == 0");
    if (l->max_seq_len < 0 || l->max_seq_len > hstu::kMaxSeqLen)
        return fail(HSTU_ERR_ARG, "max_seq_len %d outside [0, %d]", l->max_seq_len, hstu::kMaxSeqLen);
    if (l->num_rows < 0) return fail(HSTU_ERR_ARG, "num_rows < 0");
    if (int64_t(l->max_seq_len) * 4 * l->H * l->d * 2 > int64_t(0x7fffffff))
        return fail(HSTU_ERR_UNSUPPORTED, "max_seq_len * Z row bytes must stay below 2^31");
    if (l->num_pos_buckets < 1 || l->num_pos_buckets > hstu::kMaxPosBuckets)
        return fail(HSTU_ERR_ARG, "num_pos_buckets outside [1, %d]", hstu::kMaxPosBuckets);
    if (l->num_time_buckets < 1) return fail(HSTU_ERR_ARG, "num_time_buckets < 1");
    if (!std::isfinite(l->alpha)) return fail(HSTU_ERR_ARG, "alpha is not finite");
    if (!(l->ln_eps > 0.0f) || !std::isfinite(l->ln_eps)) return fail(HSTU_ERR_ARG, "ln_eps must be > 0");
    if (l->B > 0) {
        if (!l->seq_offsets || !l->x || !l->w1 || (f2 && (!l->w2 || !l->x_out)) || !l->timestamps ||
            !l->rab_pos || !l->rab_time)
            return fail(HSTU_ERR_ARG, "a required pointer is NULL");
        if (!aligned16(l->x) || !aligned16(l->w1) || (f2 && (!aligned16(l->w2) || !aligned16(l->x_out))))
            return fail(HSTU_ERR_UNSUPPORTED, "layer buffers must be 16-byte aligned");
    }
    return HSTU_OK;
}

// The attention arguments of a layer whose Z (U | V | Q | K), O and Y sit in
// the given buffers.
hstu_attn_args layer_attn_args(const hstu_layer_args* l, uint16_t* z, uint16_t* o, uint16_t* y) {
    const int hd = l->H * l->d;
    hstu_attn_args a;
    memset(&a, 0, sizeof(a));
    a.struct_size = sizeof(a);
    a.B = l->B; a.H = l->H; a.d_qk = l->d; a.d_v = l->d;
    a.max_seq_len = l->max_seq_len;
    a.num_rows = l->num_rows;
    a.seq_offsets = l->seq_offsets;
    a.num_candidates = l->num_candidates;
    a.dtype = HSTU_BF16;
    a.act = HSTU_ACT_SILU;
    a.u = z;              a.u_stride = 4 * hd;
    a.v = z + 1 * hd;     a.v_stride = 4 * hd;
    a.q = z + 2 * hd;     a.q_stride = 4 * hd;
    a.k = z + 3 * hd;     a.k_stride = 4 * hd;
    a.timestamps = l->timestamps;
    a.rab_pos = l->rab_pos; a.num_pos_buckets = l->num_pos_buckets;
    a.rab_time = l->rab_time; a.num_time_buckets = l->num_time_buckets;
    a.alpha = l->alpha;
    a.o = o; a.o_stride = hd;
    a.y = y; a.y_stride = hd;
    a.ln_eps = l->ln_eps;
    return a;
}

struct LayerWs {
    size_t z, o, y, sched, total;
};

hstu_status validate_mfalcon_layer(const hstu_mfalcon_layer_args* m) {
    if (!m) return fail(HSTU_ERR_ARG, "args is NULL");
    if (m->struct_size != sizeof(hstu_mfalcon_layer_args))
        return fail(HSTU_ERR_ARG, "struct_size %u != sizeof(hstu_mfalcon_layer_args) %zu", m->struct_size,
                    sizeof(hstu_mfalcon_layer_args));
    hstu_status st = validate_layer(&m->layer, false);
    if (st != HSTU_OK) return st;
    if (m->score_stride < 1) return fail(HSTU_ERR_ARG, "score_stride < 1");
    if (m->layer.B > 0) {
        if (!m->layer.num_candidates) return fail(HSTU_ERR_ARG, "layer.num_candidates is required");
        if (!m->w || !m->scores) return fail(HSTU_ERR_ARG, "w and scores must be non-NULL");
    }
    return HSTU_OK;
}

// Z, then O (no Y: the scores are taken in the epilogue), then the schedule.
struct MfalconLayerWs {
    size_t z, o, sched, total;
};

MfalconLayerWs mfalcon_layer_ws(const hstu_layer_args* l) {
    MfalconLayerWs w;
    const size_t T = size_t(l->num_rows);
    const size_t hd = size_t(l->H) * l->d;
    w.z = 0;
    w.o = align256(w.z + T * 4 * hd * 2);
    w.sched = align256(w.o + T * hd * 2);
    w.total = hstu::sched_layout(l->B, l->H, l->max_seq_len, hstu::kBf16TileM, l->d, l->num_rows, w.sched).bytes;
    return w;
}

LayerWs layer_ws(const hstu_layer_args* l) {
    LayerWs w;
    const size_t T = size_t(l->num_rows);
    const size_t hd = size_t(l->H) * l->d;
    w.z = 0;
    w.o = align256(w.z + T * 4 * hd * 2);
    w.y = align256(w.o + T * hd * 2);
    w.sched = align256(w.y + T * hd * 2);
    w.total = hstu::sched_layout(l->B, l->H, l->max_seq_len, hstu::kBf16TileM, l->d, l->num_rows, w.sched).bytes;
    return w;
}

// ---- layer gradients

// The attention-gradient arguments of a layer (U | V | Q | K, O, Y and the
// gradient buffers in the layer's workspace).
hstu_attn_bwd_args layer_attn_bwd_args(const hstu_layer_args* l, uint16_t* z, uint16_t* o, uint16_t* y,
                                       uint16_t* dy, uint16_t* dz, float* drp, float* drt) {
    const int hd = l->H * l->d;
    hstu_attn_bwd_args g;
    memset(&g, 0, sizeof(g));
    g.struct_size = sizeof(g);
    g.attn = layer_attn_args(l, z, o, y);
    g.attn.y = nullptr;
    g.dy = dy; g.dy_stride = hd;
    g.du = dz;              g.du_stride = 4 * hd;
    g.dv = dz + 1 * hd;     g.dv_stride = 4 * hd;
    g.dq = dz + 2 * hd;     g.dq_stride = 4 * hd;
    g.dk = dz + 3 * hd;     g.dk_stride = 4 * hd;
    g.drab_pos = drp;
    g.drab_time = drt;
    return g;
}

hstu_status validate_layer_bwd(const hstu_layer_bwd_args* g) {
    if (!g) return fail(HSTU_ERR_ARG, "args is NULL");
    if (g->struct_size != sizeof(hstu_layer_bwd_args))
        return fail(HSTU_ERR_ARG, "struct_size %u != sizeof(hstu_layer_bwd_args) %zu", g->struct_size,
                    sizeof(hstu_layer_bwd_args));
    hstu_layer_args l = g->layer;
    if (!l.x_out) l.x_out = const_cast<void*>(l.x);   // not written by the gradients
    hstu_status st = validate_layer(&l);
    if (st != HSTU_OK) return st;
    const int hd = l.H * l.d;
    if (l.D % 128 != 0 || hd % 128 != 0)
        return fail(HSTU_ERR_UNSUPPORTED, "layer gradients need D %% 128 == 0 and H*d %% 128 == 0");
    if (int64_t(l.num_rows) * 2 * std::max(4 * hd, l.D) > int64_t(0x7fffffff))
        return fail(HSTU_ERR_UNSUPPORTED, "num_rows * row bytes must stay below 2^31");
    if (l.B > 0 && l.num_rows > 0) {
        if (!g->dx_out || !g->dx || !g->dw1 || !g->dw2)
            return fail(HSTU_ERR_ARG, "dx_out, dx, dw1 and dw2 must be non-NULL");
        if (!aligned16(g->dx_out) || !aligned16(g->dx))
            return fail(HSTU_ERR_UNSUPPORTED, "dx_out and dx must be 16-byte aligned");
    }
    // the attention part's own limits (its buffers are the workspace's: a
    // stand-in address, never dereferenced, checks the rest)
    uint16_t* fake = reinterpret_cast<uint16_t*>(uintptr_t(0x10000));
    float* fakef = reinterpret_cast<float*>(uintptr_t(0x10000));
    hstu_attn_bwd_args ab = layer_attn_bwd_args(&l, fake, fake, fake, fake, fake, fakef, fakef);
    return validate_bwd(&ab);
}

struct LayerBwdWs {
    size_t z, pre, o, y, dy, dz, w1t, w2t, sched, attn, part, colsum, total;
};

// A training forward's saved activations: Z, f1's pre-activation, O, Y (bf16),
// laid out as the first four regions of the gradient workspace.
struct LayerSaved {
    size_t z, pre, o, y, total;
};

LayerSaved layer_saved(const hstu_layer_args* l) {
    const size_t T = size_t(l->num_rows);
    const size_t hd = size_t(l->H) * l->d, zw = 4 * hd;
    LayerSaved v;
    v.z = 0;
    v.pre = align256(v.z + T * zw * 2);
    v.o = align256(v.pre + T * zw * 2);
    v.y = align256(v.o + T * hd * 2);
    v.total = align256(v.y + T * hd * 2);
    return v;
}

// With `saved`, the four regions of the recomputed forward are empty (the
// gradients read the kept activations instead) and the layout starts at dY.
LayerBwdWs layer_bwd_ws(const hstu_layer_bwd_args* g, bool saved = false) {
    const hstu_layer_args* l = &g->layer;
    LayerBwdWs w;
    const size_t T = size_t(l->num_rows);
    const size_t Tf = saved ? 0 : T;
    const size_t hd = size_t(l->H) * l->d, zw = 4 * hd, D = size_t(l->D);
    w.z = 0;
    w.pre = align256(w.z + Tf * zw * 2);
    w.o = align256(w.pre + Tf * zw * 2);
    w.y = align256(w.o + Tf * hd * 2);
    w.dy = align256(w.y + Tf * hd * 2);
    w.dz = align256(w.dy + T * hd * 2);
    w.w1t = align256(w.dz + T * zw * 2);
    w.w2t = align256(w.w1t + D * zw * 2);
    w.sched = align256(w.w2t + hd * D * 2);
    const size_t sched_end = hstu::sched_layout(l->B, l->H, l->max_seq_len, hstu::kBf16TileM, l->d, l->num_rows,
                                                w.sched).bytes;
    w.attn = align256(sched_end);
    uint16_t* fake = reinterpret_cast<uint16_t*>(uintptr_t(0x10000));   // sizes only
    float* fakef = reinterpret_cast<float*>(uintptr_t(0x10000));
    hstu_attn_bwd_args ab = layer_attn_bwd_args(l, fake, fake, fake, fake, fake, fakef, fakef);
    w.part = align256(w.attn + bwd_ws(&ab).total);
    const size_t p1 = size_t(hstu::gemm_tn_splits(l->num_rows, int(zw), l->D)) * zw * D;
    const size_t p2 = size_t(hstu::gemm_tn_splits(l->num_rows, l->D, int(hd))) * D * hd;
    w.colsum = align256(w.part + sizeof(float) * std::max(p1, p2));
    w.total = align256(w.colsum + sizeof(float) * hstu::colsum_part_floats(int(std::max(zw, D))));
    return w;
}

}  // namespace

extern "C" {

size_t hstu_layer_workspace_bytes(const hstu_layer_args* l) {
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    hstu_status st = validate_layer(l);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != HSTU_OK) return 0;
    return layer_ws(l).total;
}

}  // extern "C"

namespace {

// One layer forward; with `saved`, Z, O and Y live there and f1 also writes
// its pre-activation there (what the gradients need).
hstu_status layer_fwd_run(const hstu_layer_args* l, void* ws, size_t ws_bytes, void* stream_, void* saved,
                          size_t saved_bytes) {
    hstu_status st = validate_layer(l);
    if (st != HSTU_OK) return st;
    if (l->B == 0 || l->num_rows == 0) return ok();
    if (validate_env()) {
        st = device_check_batch(l->B, l->num_rows, l->max_seq_len, l->seq_offsets, nullptr,
                                l->num_candidates, static_cast<hipStream_t>(stream_), true);
        if (st != HSTU_OK) return st;
    }
    const LayerWs lw = layer_ws(l);
    st = check_workspace(ws, ws_bytes, lw.total);
    if (st != HSTU_OK) return st;
    const LayerSaved sv = layer_saved(l);
    if (saved) {
        st = check_workspace(saved, saved_bytes, sv.total);
        if (st != HSTU_OK) return st;
    }
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    uint8_t* w = static_cast<uint8_t*>(ws);
    uint8_t* sb = static_cast<uint8_t*>(saved);
    const int hd = l->H * l->d;
    uint16_t* z = reinterpret_cast<uint16_t*>(saved ? sb + sv.z : w + lw.z);
    uint16_t* o = reinterpret_cast<uint16_t*>(saved ? sb + sv.o : w + lw.o);
    uint16_t* y = reinterpret_cast<uint16_t*>(saved ? sb + sv.y : w + lw.y);

    // f1 + SiLU: Z = SiLU(X W1^T + b1) -> U | V | Q | K
    hstu::GemmArgs g1;
    g1.M = l->num_rows; g1.N = 4 * hd; g1.K = l->D;
    g1.a = l->x; g1.lda = l->D;
    g1.b = l->w1; g1.ldb = l->D;
    g1.bias = l->b1;
    g1.residual = nullptr; g1.ldr = 0;
    g1.c = z; g1.ldc = 4 * hd;
    g1.silu = 1;
    if (saved) {
        g1.c_pre = sb + sv.pre;
        g1.ldcp = 4 * hd;
    }
    hipError_t e = hstu::launch_gemm_bf16(g1, stream);
    if (e != hipSuccess) return device_error(e, "f1 launch");

    hstu_attn_args a = layer_attn_args(l, z, o, y);
    Sched s = carve_sched(&a, ws, lw.sched);
    e = run_sched(&a, s, stream);
    if (e != hipSuccess) return device_error(e, "scheduler launch");
    e = run_core(&a, s, stream);
    if (e != hipSuccess) return device_error(e, "attention launch");
    e = run_ln_gate(&a, s, nullptr, nullptr, 0, false, stream);
    if (e != hipSuccess) return device_error(e, "epilogue launch");

    // f2 + residual: X_out = X + Y W2^T + b2
    hstu::GemmArgs g2;
    g2.M = l->num_rows; g2.N = l->D; g2.K = hd;
    g2.a = y; g2.lda = hd;
    g2.b = l->w2; g2.ldb = hd;
    g2.bias = l->b2;
    g2.residual = l->x; g2.ldr = l->D;
    g2.c = l->x_out; g2.ldc = l->D;
    g2.silu = 0;
    e = hstu::launch_gemm_bf16(g2, stream);
    if (e != hipSuccess) return device_error(e, "f2 launch");
    return ok();
}

}  // namespace

extern "C" {

hstu_status hstu_layer_fwd(const hstu_layer_args* l, void* ws, size_t ws_bytes, void* stream) {
    return layer_fwd_run(l, ws, ws_bytes, stream, nullptr, 0);
}

size_t hstu_layer_saved_bytes(const hstu_layer_args* l) {
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    hstu_status st = validate_layer(l);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != HSTU_OK) return 0;
    return layer_saved(l).total;
}

hstu_status hstu_layer_fwd_saved(const hstu_layer_args* l, void* saved, size_t saved_bytes, void* ws,
                                 size_t ws_bytes, void* stream) {
    if (l && l->struct_size == sizeof(hstu_layer_args) && l->B > 0 && l->num_rows > 0) {
        if (!saved) return fail(HSTU_ERR_ARG, "saved is NULL");
        // the gradients read X again (dW1 = dP^T X), and the saved buffer does
        // not keep it: X_out written over X would corrupt them silently
        const size_t xb = size_t(l->num_rows) * size_t(l->D) * 2;
        const uintptr_t x0 = uintptr_t(l->x), o0 = uintptr_t(l->x_out);
        if (l->x && l->x_out && x0 < o0 + xb && o0 < x0 + xb)
            return fail(HSTU_ERR_ARG, "x_out must not overlap x in a training forward (the gradients read x)");
    }
    return layer_fwd_run(l, ws, ws_bytes, stream, saved, saved_bytes);
}

size_t hstu_mfalcon_layer_workspace_bytes(const hstu_mfalcon_layer_args* m) {
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    hstu_status st = validate_mfalcon_layer(m);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != HSTU_OK) return 0;
    return mfalcon_layer_ws(&m->layer).total;
}

hstu_status mfalcon_layer_score(const hstu_mfalcon_layer_args* m, void* ws, size_t ws_bytes, void* stream_) {
    hstu_status st = validate_mfalcon_layer(m);
    if (st != HSTU_OK) return st;
    const hstu_layer_args* l = &m->layer;
    if (l->B == 0 || l->num_rows == 0) return ok();
    const MfalconLayerWs lw = mfalcon_layer_ws(l);
    st = check_workspace(ws, ws_bytes, lw.total);
    if (st != HSTU_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    uint8_t* w = static_cast<uint8_t*>(ws);
    const int hd = l->H * l->d;
    uint16_t* z = reinterpret_cast<uint16_t*>(w + lw.z);
    uint16_t* o = reinterpret_cast<uint16_t*>(w + lw.o);

    // f1 + SiLU over every row: the candidates read the history's K and V
    hstu::GemmArgs g1;
    g1.M = l->num_rows; g1.N = 4 * hd; g1.K = l->D;
    g1.a = l->x; g1.lda = l->D;
    g1.b = l->w1; g1.ldb = l->D;
    g1.bias = l->b1;
    g1.residual = nullptr; g1.ldr = 0;
    g1.c = z; g1.ldc = 4 * hd;
    g1.silu = 1;
    hipError_t e = hstu::launch_gemm_bf16(g1, stream);
    if (e != hipSuccess) return device_error(e, "f1 launch");

    hstu_attn_args a = layer_attn_args(l, z, o, nullptr);
    const bool cand_only = m->candidates_only != 0;
    Sched s = carve_sched(&a, ws, lw.sched);
    e = run_sched(&a, s, stream, cand_only);
    if (e != hipSuccess) return device_error(e, "scheduler launch");
    e = run_core(&a, s, stream);
    if (e != hipSuccess) return device_error(e, "attention launch");
    e = run_ln_gate(&a, s, m->w, m->scores, m->score_stride, cand_only, stream);
    if (e != hipSuccess) return device_error(e, "epilogue launch");
    return ok();
}

size_t hstu_mfalcon_cached_workspace_bytes(const hstu_mfalcon_cached_args* m) {
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    hstu_status st = validate_cached(m);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != HSTU_OK) return 0;
    return cached_ws(m).total;
}

hstu_status mfalcon_score_cached(const hstu_mfalcon_cached_args* m, void* ws, size_t ws_bytes, void* stream_) {
    hstu_status st = validate_cached(m);
    if (st != HSTU_OK) return st;
    if (m->B == 0 || m->num_cand_rows == 0) return ok();
    const CachedWs w = cached_ws(m);
    st = check_workspace(ws, ws_bytes, w.total);
    if (st != HSTU_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    uint8_t* wb = static_cast<uint8_t*>(ws);
    const Sched sc = carve_layout(w.cand, ws);
    float* partial = reinterpret_cast<float*>(wb + w.cand.off_part);
    int32_t* rowmap = reinterpret_cast<int32_t*>(wb + w.cand.off_rowmap);
    uint32_t* kstats = reinterpret_cast<uint32_t*>(wb + w.kstats);
    uint32_t* kenc = reinterpret_cast<uint32_t*>(wb + w.kenc);
    void* o = m->o ? m->o : static_cast<void*>(wb + w.o);
    const int64_t o_stride = m->o ? m->o_stride : int64_t(m->H) * m->d;

    // history codes (relative to each history's first event)
    hstu::SchedArgs ha;
    ha.B = m->B;
    ha.max_seq_len = m->max_hist_len;
    ha.cap = 0; ha.cap_pieces = 0;
    ha.cand_only = 0; ha.kv_mode = 0; ha.H = m->H; ha.slots = 0; ha.part_slots = 0;
    ha.split = nullptr;
    ha.offsets = m->hist_offsets; ha.lengths = nullptr; ha.ncand = nullptr;
    ha.tile_m = hstu::kBf16TileM; ha.tile_n = hstu::kBf16TileN;
    ha.ctrl = nullptr; ha.qscan = nullptr; ha.items = nullptr;
    ha.ts = m->ts_hist; ha.enc = kenc; ha.stats = kstats;
    ha.nblk = w.nblk_k; ha.cap_blk = int64_t(m->B) * w.nblk_k;
    ha.skip_list = 1;
    hipError_t e = ha.cap_blk > 0 ? hstu::launch_sched(ha, stream) : hipSuccess;
    if (e != hipSuccess) return device_error(e, "history code launch");

    // the candidates' work list (all history tiles per row block, split when
    // long) and their codes relative to the history's first event
    hstu::SchedArgs ca;
    ca.B = m->B;
    ca.max_seq_len = std::max(m->max_cands, m->max_hist_len);
    ca.cap = (int64_t)w.cand.cap; ca.cap_pieces = (int64_t)w.cand.cap_pieces;
    ca.cand_only = 0; ca.kv_mode = 0; ca.H = m->H;
    ca.slots = hstu::attn_bf16_slots(); ca.part_slots = w.cand.part_slots;
    ca.split = sc.split;
    ca.offsets = m->cand_offsets; ca.lengths = nullptr; ca.ncand = nullptr;
    ca.tile_m = hstu::kBf16TileM; ca.tile_n = hstu::kBf16TileN;
    ca.ctrl = sc.ctrl; ca.qscan = sc.qscan; ca.items = sc.items; ca.item_seq = nullptr;
    ca.ts = m->ts_cand; ca.enc = sc.enc; ca.stats = sc.stats;
    ca.nblk = w.cand.nblk; ca.cap_blk = (int64_t)w.cand.cap_blk;
    ca.kv_offsets = m->hist_offsets; ca.ref_offsets = m->hist_offsets; ca.ref_ts = m->ts_hist;
    e = hstu::launch_sched(ca, stream);
    if (e != hipSuccess) return device_error(e, "scheduler launch");

    hstu::AttnCoreArgs c;
    c.H = m->H; c.d = m->d;
    c.offsets = m->hist_offsets; c.lengths = nullptr; c.ncand = nullptr;
    c.q = m->q; c.q_stride = m->q_stride;
    c.k = m->k_hist; c.k_stride = m->k_hist_stride;
    c.v = m->v_hist; c.v_stride = m->v_hist_stride;
    c.ts = m->ts_hist;
    c.rab_pos = m->rab_pos; c.P = m->num_pos_buckets; c.rp_head_stride = m->rab_pos_head_stride;
    c.rab_time = m->rab_time; c.NT = m->num_time_buckets; c.rt_head_stride = m->rab_time_head_stride;
    c.alpha = m->alpha; c.act = HSTU_ACT_SILU;
    c.o = o; c.o_stride = o_stride;
    c.items = sc.items; c.ctrl = sc.ctrl; c.cursor = sc.ctrl + 1;
    c.partial = partial; c.rowmap = rowmap;
    c.nblk = w.nblk_k; c.stats = kstats; c.enc = kenc; c.num_rows = m->num_hist_rows;
    c.ev_begin = static_cast<hipEvent_t>(m->ev_core_begin);
    c.ev_end = static_cast<hipEvent_t>(m->ev_core_end);
    c.q_offsets = m->cand_offsets; c.ts_q = m->ts_cand; c.enc_q = sc.enc; c.stats_q = sc.stats;
    c.nblk_q = w.cand.nblk;
    e = hstu::launch_attn_bf16(c, stream);
    if (e != hipSuccess) return device_error(e, "attention launch");

    hstu::LnGateArgs l;
    l.B = m->B; l.num_rows = m->num_cand_rows; l.width = m->H * m->d; l.dtype = HSTU_BF16;
    l.offsets = m->cand_offsets; l.lengths = nullptr; l.ncand = nullptr;
    l.o = o; l.o_stride = o_stride;
    l.u = m->u; l.u_stride = m->u_stride;
    l.y = nullptr; l.y_stride = 0;
    l.eps = m->ln_eps;
    l.w = m->w; l.scores = m->scores; l.score_stride = m->score_stride;
    l.rowmap = rowmap; l.partial = partial; l.H = m->H; l.d = m->d; l.BM = hstu::kBf16TileM; l.cand_only = 0;
    l.cross = 1;
    l.sq = m->q; l.sqs = m->q_stride;
    l.sk = m->k; l.sks = m->k_stride;
    l.sv = m->v; l.svs = m->v_stride;
    l.rab_pos = m->rab_pos; l.rp_hs = m->rab_pos_head_stride;
    l.rab_time = m->rab_time; l.rt_hs = m->rab_time_head_stride;
    l.alpha = m->alpha;
    e = hstu::launch_ln_gate(l, stream);
    if (e != hipSuccess) return device_error(e, "epilogue launch");
    return ok();
}

size_t hstu_layer_bwd_workspace_bytes(const hstu_layer_bwd_args* g) {
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    hstu_status st = validate_layer_bwd(g);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != HSTU_OK) return 0;
    return layer_bwd_ws(g).total;
}

size_t hstu_layer_bwd_saved_workspace_bytes(const hstu_layer_bwd_args* g) {
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    hstu_status st = validate_layer_bwd(g);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != HSTU_OK) return 0;
    return layer_bwd_ws(g, true).total;
}

}  // extern "C"

namespace {

// Layer gradients; with `saved` (a training forward's activations) Z, its
// pre-activation, O and Y are read from there instead of recomputed.
hstu_status layer_bwd_run(const hstu_layer_bwd_args* g, void* ws, size_t ws_bytes, void* stream_,
                          const void* saved, size_t saved_bytes) {
    hstu_status st = validate_layer_bwd(g);
    if (st != HSTU_OK) return st;
    const hstu_layer_args* l = &g->layer;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (l->B > 0 && l->num_rows > 0 && validate_env()) {
        st = device_check_batch(l->B, l->num_rows, l->max_seq_len, l->seq_offsets, nullptr, l->num_candidates,
                                stream, true);
        if (st != HSTU_OK) return st;
    }
    if (l->B == 0 || l->num_rows == 0) {   // empty batch: zero parameter gradients
        const size_t zw4 = size_t(4) * l->H * l->d;
        hipError_t e = hipSuccess;
        auto clear = [&](void* p, size_t bytes) {
            if (p && e == hipSuccess) e = hipMemsetAsync(p, 0, bytes, stream);
        };
        clear(g->dw1, sizeof(float) * zw4 * l->D);
        clear(g->db1, sizeof(float) * zw4);
        clear(g->dw2, sizeof(float) * size_t(l->D) * l->H * l->d);
        clear(g->db2, sizeof(float) * l->D);
        clear(g->drab_pos, sizeof(float) * l->num_pos_buckets);
        clear(g->drab_time, sizeof(float) * l->num_time_buckets);
        return e == hipSuccess ? ok() : device_error(e, "clearing the gradients");
    }
    const LayerBwdWs lw = layer_bwd_ws(g, saved != nullptr);
    st = check_workspace(ws, ws_bytes, lw.total);
    if (st != HSTU_OK) return st;
    uint8_t* w = static_cast<uint8_t*>(ws);
    const int hd = l->H * l->d, zw = 4 * hd, D = l->D;
    const int64_t T = l->num_rows;
    uint16_t* z = reinterpret_cast<uint16_t*>(w + lw.z);
    uint16_t* pre = reinterpret_cast<uint16_t*>(w + lw.pre);
    uint16_t* o = reinterpret_cast<uint16_t*>(w + lw.o);
    uint16_t* y = reinterpret_cast<uint16_t*>(w + lw.y);
    if (saved) {
        const LayerSaved sv = layer_saved(l);
        st = check_workspace(const_cast<void*>(saved), saved_bytes, sv.total);
        if (st != HSTU_OK) return st;
        // (read only below: the gradients never write the saved activations)
        uint8_t* sb = static_cast<uint8_t*>(const_cast<void*>(saved));
        z = reinterpret_cast<uint16_t*>(sb + sv.z);
        pre = reinterpret_cast<uint16_t*>(sb + sv.pre);
        o = reinterpret_cast<uint16_t*>(sb + sv.o);
        y = reinterpret_cast<uint16_t*>(sb + sv.y);
    }
    uint16_t* dy = reinterpret_cast<uint16_t*>(w + lw.dy);
    uint16_t* dz = reinterpret_cast<uint16_t*>(w + lw.dz);
    uint16_t* w1t = reinterpret_cast<uint16_t*>(w + lw.w1t);
    uint16_t* w2t = reinterpret_cast<uint16_t*>(w + lw.w2t);
    float* part = reinterpret_cast<float*>(w + lw.part);
    float* cpart = reinterpret_cast<float*>(w + lw.colsum);

    hipError_t e = hipSuccess;
    if (!saved) {
        // forward recomputation: Z and its pre-activation, then O and Y
        hstu::GemmArgs g1;
        g1.M = T; g1.N = zw; g1.K = D;
        g1.a = l->x; g1.lda = D;
        g1.b = l->w1; g1.ldb = D;
        g1.bias = l->b1;
        g1.residual = nullptr; g1.ldr = 0;
        g1.c = z; g1.ldc = zw;
        g1.silu = 1;
        g1.c_pre = pre; g1.ldcp = zw;
        e = hstu::launch_gemm_bf16(g1, stream);
        if (e != hipSuccess) return device_error(e, "f1 launch");
        hstu_attn_args a = layer_attn_args(l, z, o, y);
        Sched s = carve_sched(&a, ws, lw.sched);
        e = run_sched(&a, s, stream);
        if (e == hipSuccess) e = run_core(&a, s, stream);
        if (e == hipSuccess) e = run_ln_gate(&a, s, nullptr, nullptr, 0, false, stream);
        if (e != hipSuccess) return device_error(e, "attention launch");
    }

    // f2: dY = dX_out W2 (through W2^T), dW2 = dX_out^T Y, db2 = sum_t dX_out
    e = hstu::launch_transpose(l->w2, D, hd, w2t, stream);
    if (e == hipSuccess) e = hstu::launch_transpose(l->w1, zw, D, w1t, stream);
    if (e != hipSuccess) return device_error(e, "transpose launch");
    hstu::GemmArgs gy;
    gy.M = T; gy.N = hd; gy.K = D;
    gy.a = g->dx_out; gy.lda = D;
    gy.b = w2t; gy.ldb = D;
    gy.bias = nullptr;
    gy.residual = nullptr; gy.ldr = 0;
    gy.c = dy; gy.ldc = hd;
    gy.silu = 0;
    e = hstu::launch_gemm_bf16(gy, stream);
    if (e != hipSuccess) return device_error(e, "dY launch");
    hstu::GemmTnArgs t2;
    t2.a = g->dx_out; t2.lda = D;
    t2.b = y; t2.ldb = hd;
    t2.T = T; t2.M = D; t2.N = hd;
    t2.splits = hstu::gemm_tn_splits(T, D, hd);
    t2.part = part;
    t2.c = g->dw2;
    e = hstu::launch_gemm_tn(t2, stream);
    if (e == hipSuccess && g->db2) e = hstu::launch_colsum(g->dx_out, D, T, D, cpart, g->db2, stream);
    if (e != hipSuccess) return device_error(e, "dW2 launch");

    // gate and attention: dU | dV | dQ | dK into dZ
    hstu_attn_bwd_args ab = layer_attn_bwd_args(l, z, o, y, dy, dz, g->drab_pos, g->drab_time);
    st = hstu_attn_bwd(&ab, w + lw.attn, lw.part - lw.attn, stream);
    if (st != HSTU_OK) return st;

    // f1 + SiLU: dP = dZ SiLU'(P), dX = dX_out + dP W1, dW1 = dP^T X, db1 = sum_t dP
    e = hstu::launch_silu_grad(dz, pre, T * zw, stream);
    if (e != hipSuccess) return device_error(e, "SiLU slope launch");
    hstu::GemmTnArgs t1;
    t1.a = dz; t1.lda = zw;
    t1.b = l->x; t1.ldb = D;
    t1.T = T; t1.M = zw; t1.N = D;
    t1.splits = hstu::gemm_tn_splits(T, zw, D);
    t1.part = part;
    t1.c = g->dw1;
    e = hstu::launch_gemm_tn(t1, stream);
    if (e == hipSuccess && g->db1) e = hstu::launch_colsum(dz, zw, T, zw, cpart, g->db1, stream);
    if (e != hipSuccess) return device_error(e, "dW1 launch");
    hstu::GemmArgs gx;
    gx.M = T; gx.N = D; gx.K = zw;
    gx.a = dz; gx.lda = zw;
    gx.b = w1t; gx.ldb = zw;
    gx.bias = nullptr;
    gx.residual = g->dx_out; gx.ldr = D;
    gx.c = g->dx; gx.ldc = D;
    gx.silu = 0;
    e = hstu::launch_gemm_bf16(gx, stream);
    if (e != hipSuccess) return device_error(e, "dX launch");
    return ok();
}

}  // namespace

extern "C" {

hstu_status hstu_layer_bwd(const hstu_layer_bwd_args* g, void* ws, size_t ws_bytes, void* stream) {
    return layer_bwd_run(g, ws, ws_bytes, stream, nullptr, 0);
}

hstu_status hstu_layer_bwd_saved(const hstu_layer_bwd_args* g, const void* saved, size_t saved_bytes, void* ws,
                                 size_t ws_bytes, void* stream) {
    if (g && g->struct_size == sizeof(hstu_layer_bwd_args) && g->layer.B > 0 && g->layer.num_rows > 0 && !saved)
        return fail(HSTU_ERR_ARG, "saved is NULL");
    return layer_bwd_run(g, ws, ws_bytes, stream, saved, saved_bytes);
}

size_t hstu_attn_bwd_workspace_bytes(const hstu_attn_bwd_args* g) {
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    hstu_status st = validate_bwd(g);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != HSTU_OK) return 0;
    return bwd_ws(g).total;
}

hstu_status hstu_attn_bwd(const hstu_attn_bwd_args* g, void* ws, size_t ws_bytes, void* stream_) {
    hstu_status st = validate_bwd(g);
    if (st != HSTU_OK) return st;
    const hstu_attn_args* a = &g->attn;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const int P = a->num_pos_buckets, NT = a->num_time_buckets;
    if (a->B == 0) {   // empty batch: zero table gradients
        const int hp = a->rab_pos_head_stride > 0 ? a->H : 1, ht = a->rab_time_head_stride > 0 ? a->H : 1;
        hipError_t e = hipSuccess;
        if (g->drab_pos) e = hipMemsetAsync(g->drab_pos, 0, sizeof(float) * size_t(hp) * P, stream);
        if (e == hipSuccess && g->drab_time) e = hipMemsetAsync(g->drab_time, 0, sizeof(float) * size_t(ht) * NT, stream);
        return e == hipSuccess ? ok() : device_error(e, "clearing the table gradients");
    }
    st = maybe_check_batch(a, stream);
    if (st != HSTU_OK) return st;
    const BwdWs w = bwd_ws(g);
    st = check_workspace(ws, ws_bytes, w.total);
    if (st != HSTU_OK) return st;
    uint8_t* wb = static_cast<uint8_t*>(ws);
    const Sched sq = carve_layout(w.q, ws);
    const Sched skv = carve_layout(w.kv, ws);
    const int hd = a->H * a->d_v;
    hipError_t e;

    // upstream gradient of O
    const void* dout = g->dout;
    int64_t dout_stride = g->dout_stride;
    if (g->dy) {
        hstu::LnGateBwdArgs l;
        l.B = a->B;
        l.num_rows = a->num_rows;
        l.width = hd;
        l.offsets = a->seq_offsets;
        l.lengths = a->seq_lengths;
        l.o = a->o; l.o_stride = a->o_stride;
        l.u = a->u; l.u_stride = a->u_stride;
        l.dy = g->dy; l.dy_stride = g->dy_stride;
        l.dout = wb + w.dout; l.dout_stride = hd;
        l.du = g->du; l.du_stride = g->du_stride;
        l.eps = a->ln_eps;
        e = hstu::launch_ln_gate_bwd(l, stream);
        if (e != hipSuccess) return device_error(e, "gate gradient launch");
        dout = wb + w.dout;
        dout_stride = hd;
    }

    // work lists: query-major (no split pieces) with the timestamp codes,
    // then key-major
    hstu::SchedArgs qa = make_sched_args(a, sq, false);
    qa.slots = 0;
    qa.part_slots = 0;
    hstu::SchedArgs ka = make_sched_args(a, skv, false);
    ka.kv_mode = 1;
    ka.slots = 0;
    ka.part_slots = 0;
    ka.enc = nullptr;
    ka.cap_blk = 0;
    e = hstu::launch_sched_pair(qa, ka, reinterpret_cast<int64_t*>(wb + w.gbase), stream);
    if (e != hipSuccess) return device_error(e, "scheduler launch");

    hstu::AttnBwdArgs b;
    b.H = a->H;
    b.offsets = a->seq_offsets; b.lengths = a->seq_lengths; b.ncand = a->num_candidates;
    b.q = a->q; b.q_stride = a->q_stride;
    b.k = a->k; b.k_stride = a->k_stride;
    b.v = a->v; b.v_stride = a->v_stride;
    b.dout = dout; b.dout_stride = dout_stride;
    b.ts = a->timestamps;
    b.rab_pos = a->rab_pos; b.P = P; b.rp_head_stride = a->rab_pos_head_stride;
    b.rab_time = a->rab_time; b.NT = NT; b.rt_head_stride = a->rab_time_head_stride;
    b.alpha = a->alpha;
    b.act = a->act;
    b.dq = g->dq; b.dq_stride = g->dq_stride;
    b.dk = g->dk; b.dk_stride = g->dk_stride;
    b.dv = g->dv; b.dv_stride = g->dv_stride;
    b.drab_pos = g->drab_pos; b.drab_time = g->drab_time;
    b.q_items = sq.items; b.q_ctrl = sq.ctrl;
    b.kv_items = skv.items; b.kv_ctrl = skv.ctrl;
    b.nblk = w.q.nblk;
    b.stats = sq.stats;
    b.enc = sq.enc;
    b.num_rows = a->num_rows;
    b.rab_part = reinterpret_cast<float*>(wb + w.part);
    b.rab_part2 = reinterpret_cast<float*>(wb + w.part2);
    b.gbase = reinterpret_cast<int64_t*>(wb + w.gbase);
    b.gbuf = reinterpret_cast<float*>(wb + w.gbuf);
    b.gcap = w.gcap;
    b.kp = wb + w.kp;
    b.B = a->B;
    b.ev_dq_begin = static_cast<hipEvent_t>(g->ev_dq_begin);
    b.ev_dq_end = static_cast<hipEvent_t>(g->ev_dq_end);
    b.ev_dkv_begin = static_cast<hipEvent_t>(g->ev_dkv_begin);
    b.ev_dkv_end = static_cast<hipEvent_t>(g->ev_dkv_end);
    e = hstu::launch_attn_bwd(b, stream);
    if (e != hipSuccess) return device_error(e, "gradient kernels launch");
    return ok();
}

hstu_status hstu_stochastic_length(const hstu_sl_args* a, void* stream_) {
    if (!a) return fail(HSTU_ERR_ARG, "args is NULL");
    if (a->struct_size != sizeof(hstu_sl_args))
        return fail(HSTU_ERR_ARG, "struct_size %u != sizeof(hstu_sl_args) %zu", a->struct_size, sizeof(hstu_sl_args));
    if (a->B < 0 || a->num_rows < 0) return fail(HSTU_ERR_ARG, "B and num_rows must be >= 0");
    if (!a->caps && a->cap < 0) return fail(HSTU_ERR_ARG, "cap must be >= 0");
    if (a->num_tensors < 0 || a->num_tensors > HSTU_SL_MAX_TENSORS)
        return fail(HSTU_ERR_ARG, "num_tensors outside [0, %d]", HSTU_SL_MAX_TENSORS);
    if (a->B > 0 && (!a->seq_offsets || !a->out_offsets || !a->out_index))
        return fail(HSTU_ERR_ARG, "seq_offsets, out_offsets and out_index must be non-NULL");
    for (int t = 0; t < a->num_tensors; ++t) {
        if (!a->src[t] || !a->dst[t]) return fail(HSTU_ERR_ARG, "tensor %d: NULL pointer", t);
        if (a->row_bytes[t] <= 0 || a->row_bytes[t] % 4 != 0)
            return fail(HSTU_ERR_ARG, "tensor %d: row_bytes must be a positive multiple of 4", t);
        if (a->src_stride[t] < a->row_bytes[t] || a->dst_stride[t] < a->row_bytes[t] || a->src_stride[t] % 4 ||
            a->dst_stride[t] % 4)
            return fail(HSTU_ERR_ARG, "tensor %d: strides must be multiples of 4 and >= row_bytes", t);
        if ((reinterpret_cast<uintptr_t>(a->src[t]) | reinterpret_cast<uintptr_t>(a->dst[t])) & 3u)
            return fail(HSTU_ERR_ARG, "tensor %d: rows must be 4-byte aligned", t);
    }
    if (a->B == 0) return ok();
    hstu::SlArgs s;
    s.B = a->B;
    s.num_rows = a->num_rows;
    s.offsets = a->seq_offsets;
    s.cap = a->cap;
    s.caps = a->caps;
    s.seed = a->seed;
    s.step = a->step;
    s.out_offsets = a->out_offsets;
    s.out_index = a->out_index;
    s.num_tensors = a->num_tensors;
    for (int t = 0; t < hstu::kSlMaxTensors; ++t) {
        const bool used = t < a->num_tensors;
        s.src[t] = used ? a->src[t] : nullptr;
        s.src_stride[t] = used ? a->src_stride[t] : 0;
        s.dst[t] = used ? a->dst[t] : nullptr;
        s.dst_stride[t] = used ? a->dst_stride[t] : 0;
        s.row_bytes[t] = used ? a->row_bytes[t] : 0;
    }
    hipError_t e = hstu::launch_stochastic_length(s, static_cast<hipStream_t>(stream_));
    if (e != hipSuccess) return device_error(e, "stochastic length launch");
    return ok();
}

hstu_status hstu_validate_offsets(const hstu_attn_args* a, void* stream_) {
    if (!a) return fail(HSTU_ERR_ARG, "args is NULL");
    if (a->struct_size != sizeof(hstu_attn_args))
        return fail(HSTU_ERR_ARG, "struct_size %u != sizeof(hstu_attn_args) %zu", a->struct_size,
                    sizeof(hstu_attn_args));
    if (a->B < 0 || a->num_rows < 0 || a->max_seq_len < 0) return fail(HSTU_ERR_ARG, "B, num_rows and max_seq_len must be >= 0");
    if (a->B == 0) return ok();
    if (!a->seq_offsets) return fail(HSTU_ERR_ARG, "seq_offsets is NULL");
    return device_check_batch(a->B, a->num_rows, a->max_seq_len, a->seq_offsets, a->seq_lengths,
                              a->num_candidates, static_cast<hipStream_t>(stream_));
}

hstu_status hstu_attn_schedule(const hstu_attn_args* a, void* ws, size_t ws_bytes, int32_t* items_out,
                               int64_t cap, int64_t* count_out, int32_t* tile_m_out, int32_t* tile_n_out,
                               void* stream_) {
    hstu_status st = validate_attn(a, false);
    if (st != HSTU_OK) return st;
    if (!count_out) return fail(HSTU_ERR_ARG, "count_out is NULL");
    if (tile_m_out) *tile_m_out = tile_m_for(a->dtype);
    if (tile_n_out) *tile_n_out = tile_n_for(a->dtype);
    *count_out = 0;
    if (a->B == 0) return ok();
    const size_t need = sched_layout_for(a, 0).bytes;
    st = check_workspace(ws, ws_bytes, need);
    if (st != HSTU_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    Sched s = carve_sched(a, ws, 0);
    hipError_t e = run_sched(a, s, stream);
    if (e != hipSuccess) return device_error(e, "scheduler launch");
    int32_t count = 0;
    e = hipMemcpyAsync(&count, s.ctrl, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return device_error(e, "reading the item count");
    *count_out = count;
    const int64_t n = count < cap ? count : cap;
    if (n > 0 && items_out) {
        e = hipMemcpyAsync(items_out, s.items, size_t(n) * sizeof(hstu::WorkItem), hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return device_error(e, "reading the work list");
    }
    return ok();
}

}  // extern "C"
