// api.hip -- the C ABI of libatomattn.so (declared in include/atom_attn.h):
// argument checks, workspace layout, weight packing jobs and the launch
// sequence of one block call. Host code only; every step of the block runs
// in the kernels of pack/prep/slot/post.hip.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/atom_attn.h"
#include "kernels.hpp"

using namespace waa;

namespace {

constexpr int kAbiVersion = 6;

// ------------------------------------------------------------ profiler

struct ProfRec {
    int kernel;
    hipEvent_t start, stop;
};
struct Profiler {
    bool on = false;
    std::vector<ProfRec> recs;
    std::vector<hipEvent_t> pool;
    const char *names[32] = {"pack", "token_proj", "prep", "slot_attention",
                             "post", "pool", "masks", "s2p_token", "s2p_pair",
                             "window", "tied_bias", "tied_proj", "tied_logits",
                             "tied_softmax", "tied_out", "bwd_recompute", "bwd_slot_fwd",
                             "bwd_slot_q", "bwd_slot_kv", "bwd_chain", "slot_gather"};
    int nnames = 21;
};
Profiler g_prof;

} // namespace

namespace waa {
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

void allow_lds(const void *fn, size_t bytes) {
    static std::mutex mu;
    static std::unordered_map<const void *, size_t> limit;
    std::lock_guard<std::mutex> lock(mu);
    size_t &cur = limit[fn];
    if (bytes > cur &&
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess)
        cur = bytes;
}
} // namespace waa

namespace {

hipEvent_t prof_event() {
    if (!g_prof.pool.empty()) {
        hipEvent_t e = g_prof.pool.back();
        g_prof.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    // timing-only events: no system-scope fence (no cache writeback and
    // invalidate between the kernels they bracket)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess)
        return nullptr;
    return e;
}

enum { KN_PACK = 0, KN_TOKEN = 1, KN_PREP = 2, KN_SLOT = 3, KN_POST = 4, KN_POOL = 5, KN_MASKS = 6 };
static_assert(KN_MASKS + 1 == waa::KN_S2P_TOK, "profiler ids of the other operators follow");

// Run one launcher, bracketed by events when profiling is on.
template <typename F> int timed(int kernel, hipStream_t s, F launch) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (g_prof.on) {
        e0 = prof_event();
        e1 = prof_event();
        if (e0 && e1)
            (void)hipEventRecord(e0, s);
    }
    hipError_t err = launch();
    if (g_prof.on && e0 && e1) {
        (void)hipEventRecord(e1, s);
        g_prof.recs.push_back({kernel, e0, e1});
    }
    return err == hipSuccess ? ATOM_ATTN_OK : ATOM_ATTN_ELAUNCH;
}

} // namespace

namespace waa {
ProfSpan prof_begin(int kernel, hipStream_t s) {
    ProfSpan sp;
    sp.kernel = kernel;
    if (g_prof.on) {
        sp.e0 = prof_event();
        sp.e1 = prof_event();
        if (sp.e0 && sp.e1)
            (void)hipEventRecord(sp.e0, s);
    }
    return sp;
}
void prof_end(const ProfSpan &sp, hipStream_t s) {
    if (g_prof.on && sp.e0 && sp.e1) {
        (void)hipEventRecord(sp.e1, s);
        g_prof.recs.push_back({sp.kernel, sp.e0, sp.e1});
    }
}
} // namespace waa

namespace {

// ------------------------------------------------------------ checks

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool dims_valid(const atom_attn_dims *d) {
    return d && d->B >= 1 && d->A >= 1 && d->T >= 1 && d->K >= 1 && d->C >= 1 &&
           d->S >= 1 && d->H >= 1 && d->D >= 1 && d->V >= 1 && d->M >= 1 &&
           d->U >= 1;
}

// eps must be finite and stay > 0 once represented in the input dtype.
bool eps_valid(double eps, int dtype) {
    if (!(eps > 0.0) || !std::isfinite(eps))
        return false;
    const float f = (float)eps;
    if (!(f > 0.0f) || !std::isfinite(f))
        return false;
    if (dtype == ATOM_ATTN_BF16) {
        uint32_t u;
        std::memcpy(&u, &f, 4);
        u += 0x7fffu + ((u >> 16) & 1u);
        if ((u >> 16) == 0)
            return false;
    }
    return true;
}

bool mult32_le(int64_t x, int64_t cap) { return x % 32 == 0 && x <= cap; }

// The slot kernel addresses one head's rows of the transposed V copy with
// a 32-bit byte offset from the head's base: D rows of vt_pitch(A) values.
bool vt_offsets_fit(int64_t A, int64_t D, int esz) {
    if (A > ((int64_t)1 << 30))
        return false;
    return D * (int64_t)vt_pitch((int)A) * esz < ((int64_t)1 << 31);
}

// The kernels' supported set; returns ATOM_ATTN_OK or EUNSUPPORTED.
int shape_supported(const atom_attn_dims *d, int style, int stage, int dtype) {
    const int64_t HD = d->H * d->D;
    if (!mult32_le(d->C, 512) || !mult32_le(d->S, 512) || !mult32_le(HD, 512) ||
        !mult32_le(d->M, 512) || !mult32_le(d->U, 512))
        return ATOM_ATTN_EUNSUPPORTED;
    if ((d->D != 16 && d->D != 32 && d->D != 64 && d->D != 128) || d->K > 256)
        return ATOM_ATTN_EUNSUPPORTED;
    if (d->B * d->A > (int64_t)1 << 30 || d->B * d->T > (int64_t)1 << 30 ||
        d->B * d->A * d->K > ((int64_t)1 << 31) - 1 ||
        d->B * d->H * d->A * d->K > ((int64_t)1 << 31) - 1 ||
        !vt_offsets_fit(d->A, d->D, dtype == ATOM_ATTN_BF16 ? 2 : 4))
        return ATOM_ATTN_EUNSUPPORTED;
    const Dims dd{(int)d->B, (int)d->A, (int)d->T, (int)d->K, (int)d->C, (int)d->S,
                  (int)d->H, (int)d->D, (int)d->V, (int)d->M, (int)d->U};
    if (prep_lds_bytes(dd, dtype, style, stage) > kMaxLds ||
        post_lds_bytes(dd, dtype, style) > kMaxLds ||
        !slot_supported(dd, dtype, style))
        return ATOM_ATTN_EUNSUPPORTED;
    // pooling keys (batch * T + token) are int32
    if (stage == ATOM_ATTN_ENCODER && d->B * d->T >= ((int64_t)1 << 31))
        return ATOM_ATTN_EUNSUPPORTED;
    if (stage == ATOM_ATTN_DECODER && token_proj_lds_bytes(dd, dtype) > kMaxLds)
        return ATOM_ATTN_EUNSUPPORTED;
    return ATOM_ATTN_OK;
}

// ------------------------------------------------------------ workspace

struct Layout {
    size_t packed, q, k, v, g, o, usable, tokproj, pool_sum, pool_int, pbias, vrows, wide, total;
    int64_t pack_units;
};

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Packed weight matrices of one call, in the order they are laid out.
struct Mat {
    int64_t *off;
    const void *src;
    int64_t ld;
    int kd, n;
    bool tile; // read by the 32-row tile kernels (prep, post), not k_token_proj
};

// The matrices of one call (at most kMaxPackJobs), held in place so that a
// call makes no heap allocation.
struct MatList {
    Mat m[kMaxPackJobs];
    int n = 0;
    void push_back(const Mat &x) { m[n++] = x; }
    Mat *begin() { return m; }
    Mat *end() { return m + n; }
    size_t size() const { return (size_t)n; }
    Mat &operator[](size_t i) { return m[i]; }
};

void list_mats(const atom_attn_dims *d, int style, int stage, int esz,
               const atom_attn_params *par, PackedOffsets *off, MatList *mats) {
    const int C = (int)d->C, S = (int)d->S, HD = (int)(d->H * d->D), M = (int)d->M,
              U = (int)d->U;
    auto at = [&](const void *base, int64_t elems) -> const void * {
        return base ? (const char *)base + elems * esz : nullptr;
    };
    for (int j = 0; j < 3; ++j) off->w_scale[j] = off->w_shift[j] = -1;
    for (int j = 0; j < 2; ++j) off->w_rg[j] = -1;
    for (int j = 0; j < 6; ++j) off->w_mod[j] = -1;
    off->w_q = off->w_k = off->w_v = off->w_vg = off->w_ao = -1;
    off->ff_gate = off->ff_up = off->ff_out = off->w_pool = off->w_token = -1;
    if (style == ATOM_ATTN_AF3) {
        for (int j = 0; j < 3; ++j) {
            mats->push_back({&off->w_scale[j], at(par ? par->w_scale : nullptr, (int64_t)j * S * C), C, S, C, true});
            mats->push_back({&off->w_shift[j], at(par ? par->w_shift : nullptr, (int64_t)j * S * C), C, S, C, true});
        }
        for (int j = 0; j < 2; ++j)
            mats->push_back({&off->w_rg[j], at(par ? par->w_residual_gate : nullptr, (int64_t)j * S * C), C, S, C, true});
    } else {
        for (int j = 0; j < 6; ++j)
            mats->push_back({&off->w_mod[j], at(par ? par->w_mod : nullptr, (int64_t)j * C), 6 * C, S, C, true});
    }
    mats->push_back({&off->w_q, par ? par->w_q : nullptr, HD, C, HD, true});
    mats->push_back({&off->w_k, par ? par->w_k : nullptr, HD, C, HD, true});
    mats->push_back({&off->w_v, par ? par->w_v : nullptr, HD, C, HD, true});
    mats->push_back({&off->w_vg, par ? par->w_value_gate : nullptr, HD, C, HD, true});
    mats->push_back({&off->w_ao, par ? par->w_attention_out : nullptr, C, HD, C, true});
    mats->push_back({&off->ff_gate, par ? par->w_ff_gate : nullptr, M, C, M, true});
    mats->push_back({&off->ff_up, par ? par->w_ff_up : nullptr, M, C, M, true});
    mats->push_back({&off->ff_out, par ? par->w_ff_out : nullptr, C, M, C, true});
    if (stage == ATOM_ATTN_ENCODER)
        mats->push_back({&off->w_pool, par ? par->w_pool : nullptr, U, C, U, true});
    else
        mats->push_back({&off->w_token, par ? par->w_token : nullptr, C, U, C, false});
    int64_t o = 0;
    for (auto &m : *mats) {
        *m.off = o;
        o += packed_units(m.kd, m.n, esz);
    }
}

Layout layout_of(const atom_attn_dims *d, int style, int stage, int dtype) {
    const int esz = dtype == ATOM_ATTN_BF16 ? 2 : 4;
    PackedOffsets off;
    MatList mats;
    list_mats(d, style, stage, esz, nullptr, &off, &mats);
    int64_t units = 0;
    for (auto &m : mats)
        units += packed_units(m.kd, m.n, esz);
    Layout L;
    const size_t N = (size_t)(d->B * d->A);
    const size_t rowb = (size_t)(d->H * d->D) * esz;
    const size_t row32 = (size_t)(d->H * d->D) * 4; // Q and K are fp32
    size_t o = 0;
    L.pack_units = units;
    L.packed = o; o = up256(o + (size_t)units * 16);
    L.q = o; o = up256(o + N * row32);
    L.k = o; o = up256(o + N * row32);
    // V transposed per batch: [B][H*D][vt_pitch(A)]
    L.v = o; o = up256(o + (size_t)(d->B * d->H * d->D) * vt_pitch((int)d->A) * esz);
    L.g = o; o = up256(o + N * rowb);
    L.o = o; o = up256(o + N * rowb);
    L.usable = o; o = up256(o + N);
    L.tokproj = o;
    if (stage == ATOM_ATTN_DECODER)
        o = up256(o + (size_t)(d->B * d->T * d->C) * 4);
    const size_t ntile = (N + 31) / 32;
    L.pool_sum = o;
    L.pool_int = o;
    if (stage == ATOM_ATTN_ENCODER) {
        o = up256(o + ntile * 2 * (size_t)d->U * 4);
        L.pool_int = o;
        o = up256(o + ntile * 8 * 4);
    }
    // AF3 pair bias of every slot, [N*K][4] fp32 (used when the projection
    // kernel computes it)
    L.pbias = o;
    if (style == ATOM_ATTN_AF3)
        o = up256(o + N * (size_t)d->K * 16);
    // row-major V and the queue of wide query blocks (slot gather path)
    L.vrows = o; o = up256(o + N * rowb);
    L.wide = o; o = up256(o + 4 * ((size_t)d->B * ((d->A + 15) / 16) + 1));
    L.total = o;
    return L;
}

int check_common(const atom_attn_dims *d, int style, int stage, int dtype) {
    if (!dims_valid(d))
        return ATOM_ATTN_EINVAL;
    if (style != ATOM_ATTN_AF3 && style != ATOM_ATTN_ESMFOLD2)
        return ATOM_ATTN_EINVAL;
    if (stage != ATOM_ATTN_ENCODER && stage != ATOM_ATTN_DECODER)
        return ATOM_ATTN_EINVAL;
    if (dtype != ATOM_ATTN_F32 && dtype != ATOM_ATTN_BF16)
        return ATOM_ATTN_EINVAL;
    if (style == ATOM_ATTN_ESMFOLD2 && d->D % 2 != 0)
        return ATOM_ATTN_EODD_HEAD;
    return ATOM_ATTN_OK;
}

// The weight matrices a style/stage needs are present and 16-byte aligned.
bool matrices_present(const atom_attn_params *par, int style, int stage) {
    const void *common[] = {par->w_q, par->w_k, par->w_v, par->w_value_gate,
                            par->w_attention_out, par->w_ff_gate, par->w_ff_up,
                            par->w_ff_out,
                            stage == ATOM_ATTN_ENCODER ? par->w_pool : par->w_token};
    for (const void *p : common)
        if (!p || !aligned16(p))
            return false;
    if (style == ATOM_ATTN_AF3) {
        const void *af[] = {par->w_scale, par->w_shift, par->w_residual_gate};
        for (const void *p : af)
            if (!p || !aligned16(p))
                return false;
    } else if (!par->w_mod || !aligned16(par->w_mod)) {
        return false;
    }
    return true;
}

int run_block(const atom_attn_dims *d, int style, int stage, int dtype,
              const atom_attn_inputs *in, const atom_attn_params *par,
              double eps, int64_t radius, atom_attn_outputs *out,
              void *workspace, size_t ws_bytes, void *stream) {
    int rc = check_common(d, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    if (!in || !par || !out || !eps_valid(eps, dtype) || radius < -1)
        return ATOM_ATTN_EINVAL;
    const bool af3 = style == ATOM_ATTN_AF3, enc = stage == ATOM_ATTN_ENCODER;
    // pointers each style/stage needs
    const void *need_f[] = {in->atom, in->condition, par->w_q, par->w_k, par->w_v,
                            par->w_value_gate, par->w_attention_out, par->w_ff_gate,
                            par->w_ff_up, par->w_ff_out, out->hidden, out->attention};
    for (const void *p : need_f)
        if (!p || !aligned16(p))
            return ATOM_ATTN_EINVAL;
    if (!in->valid || !in->token_valid || !in->window_mask || !in->atom_to_token ||
        !in->key_index)
        return ATOM_ATTN_EINVAL;
    if (af3) {
        const void *nf[] = {in->pair, par->cond_scale, par->w_scale, par->b_scale,
                            par->w_shift, par->w_residual_gate, par->b_residual_gate,
                            par->b_q, par->pair_scale, par->w_pair};
        for (const void *p : nf)
            if (!p || !aligned16(p))
                return ATOM_ATTN_EINVAL;
    } else {
        const void *nf[] = {in->rope_cos, in->rope_sin, par->w_mod};
        for (const void *p : nf)
            if (!p || !aligned16(p))
                return ATOM_ATTN_EINVAL;
    }
    if (enc) {
        if (!par->w_pool || !out->token_output || !aligned16(par->w_pool) ||
            !aligned16(out->token_output))
            return ATOM_ATTN_EINVAL;
    } else {
        const void *nf[] = {in->token, par->w_token, par->readout_scale, par->w_readout,
                            out->position_update};
        for (const void *p : nf)
            if (!p || !aligned16(p))
                return ATOM_ATTN_EINVAL;
        if (!af3 && !par->readout_bias)
            return ATOM_ATTN_EINVAL;
    }
    rc = shape_supported(d, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    const Layout L = layout_of(d, style, stage, dtype);
    if (!workspace || !aligned16(workspace) || ws_bytes < L.total)
        return ATOM_ATTN_EWORKSPACE;
    // weights packed beforehand by atom_attn_pack_params: both layouts, the
    // 32-column blocks first, then the 16-column strips
    const bool prepacked = par->packed != nullptr;
    if (prepacked && !aligned16(par->packed))
        return ATOM_ATTN_EINVAL;

    const int esz = dtype == ATOM_ATTN_BF16 ? 2 : 4;
    const int dt = dtype == ATOM_ATTN_BF16 ? 1 : 0;
    const int st = af3 ? STYLE_AF3 : STYLE_ESM;
    const int sg = enc ? STAGE_ENCODER : STAGE_DECODER;
    char *ws = (char *)workspace;
    hipStream_t s = (hipStream_t)stream;

    PackedOffsets off;
    MatList mats;
    list_mats(d, style, stage, esz, par, &off, &mats);
    // prep and post with eight waves (32x16 strips) when their grid has at
    // most one tile per CU; their matrices are then packed in the strip
    // layout
    const int64_t ntile = (d->B * d->A + 31) / 32;
    const bool nw8 = ntile <= device_cus();
    PackArgs pa;
    std::memset(&pa, 0, sizeof(pa));
    pa.njobs = (int)mats.size();
    for (size_t i = 0; i < mats.size(); ++i)
        pa.job[i] = PackJob{mats[i].src, mats[i].ld, mats[i].kd, mats[i].n, *mats[i].off,
                            nw8 && mats[i].tile ? 1 : 0};
    pa.total = L.pack_units;
    pa.out = (uint4 *)(ws + L.packed);

    BlockArgs a;
    std::memset(&a, 0, sizeof(a));
    a.d = Dims{(int)d->B, (int)d->A, (int)d->T, (int)d->K, (int)d->C, (int)d->S,
               (int)d->H, (int)d->D, (int)d->V, (int)d->M, (int)d->U};
    a.eps = (float)eps;
    a.radius = radius;
    a.atom = in->atom; a.condition = in->condition; a.pair = in->pair;
    a.token = in->token; a.rope_cos = in->rope_cos; a.rope_sin = in->rope_sin;
    a.valid = in->valid; a.token_valid = in->token_valid; a.window_mask = in->window_mask;
    a.atom_to_token = in->atom_to_token; a.key_index = in->key_index;
    a.cond_scale = par->cond_scale; a.b_scale = par->b_scale;
    a.b_rg = par->b_residual_gate; a.b_q = par->b_q;
    a.readout_scale = par->readout_scale; a.readout_bias = par->readout_bias;
    a.w_readout = par->w_readout;
    a.pk = prepacked ? (const uint4 *)par->packed + (nw8 ? L.pack_units : 0)
                     : (const uint4 *)(ws + L.packed);
    a.off = off;
    a.q = ws + L.q; a.k = ws + L.k; a.v = ws + L.v; a.g = ws + L.g; a.o = ws + L.o;
    a.usable = (uint8_t *)(ws + L.usable);
    a.tokproj = enc ? nullptr : (float *)(ws + L.tokproj);
    a.pool_sum = enc ? (float *)(ws + L.pool_sum) : nullptr;
    a.pool_int = enc ? (int *)(ws + L.pool_int) : nullptr;
    a.hidden = out->hidden; a.attention = out->attention;
    a.token_output = out->token_output; a.position_update = out->position_update;
    a.status = out->status;
    a.pair_scale = par->pair_scale; a.w_pair = par->w_pair;
    a.nw8 = nw8 ? 1 : 0;
    a.pbias = af3 && prep_hosts_pair_bias(a.d, dt, st, sg) ? (float *)(ws + L.pbias) : nullptr;
    a.wide = (int *)(ws + L.wide);

    SlotArgs sa;
    std::memset(&sa, 0, sizeof(sa));
    sa.B = a.d.B; sa.A = a.d.A; sa.K = a.d.K; sa.H = a.d.H; sa.D = a.d.D; sa.V = a.d.V;
    sa.eps = a.eps;
    sa.inv_sqrt_d = (float)(1.0 / std::sqrt((double)d->D));
    sa.radius = radius;
    sa.usable = a.usable; sa.window_mask = in->window_mask; sa.key_index = in->key_index;
    sa.q = a.q; sa.k = a.k; sa.v = a.v;
    sa.pair = in->pair; sa.pair_scale = par->pair_scale; sa.w_pair = par->w_pair;
    sa.pbias = a.pbias;
    sa.attention = out->attention; sa.o = a.o;
    sa.wide = a.wide; sa.vrows = ws + L.vrows; sa.vrows_out = ws + L.vrows;

    if (!prepacked &&
        (rc = timed(KN_PACK, s, [&] { return launch_pack(pa, dt, s); })) != ATOM_ATTN_OK)
        return rc;
    if (!enc && (rc = timed(KN_TOKEN, s, [&] { return launch_token_proj(a, dt, s); })) != ATOM_ATTN_OK)
        return rc;
    if ((rc = timed(KN_PREP, s, [&] { return launch_prep(a, dt, st, sg, s); })) != ATOM_ATTN_OK)
        return rc;
    if ((rc = timed(KN_SLOT, s, [&] { return launch_slot(sa, dt, st, s); })) != ATOM_ATTN_OK)
        return rc;
    if ((rc = timed(KN_SLOT_GATHER, s, [&] { return launch_slot_gather(sa, dt, st, s); })) !=
        ATOM_ATTN_OK)
        return rc;
    if ((rc = timed(KN_POST, s, [&] { return launch_post(a, dt, st, sg, s); })) != ATOM_ATTN_OK)
        return rc;
    if (enc && (rc = timed(KN_POOL, s, [&] { return launch_pool(a, dt, s); })) != ATOM_ATTN_OK)
        return rc;
    return ATOM_ATTN_OK;
}

} // namespace

namespace waa {
// Entry points for the scratch-free block call (noalloc.hip): the same
// checks and launch sequence as atom_attn_encoder/decoder.
int block_call(const atom_attn_dims *d, int style, int stage, int dtype,
               const atom_attn_inputs *in, const atom_attn_params *par, double eps,
               int64_t radius, atom_attn_outputs *out, void *workspace,
               size_t ws_bytes, void *stream) {
    return run_block(d, style, stage, dtype, in, par, eps, radius, out, workspace,
                     ws_bytes, stream);
}
int block_workspace_bytes(const atom_attn_dims *d, int style, int stage, int dtype,
                          size_t *bytes) {
    return atom_attn_workspace_bytes(d, style, stage, dtype, bytes);
}
} // namespace waa

extern "C" {

int atom_attn_version(void) { return kAbiVersion; }

const char *atom_attn_error_string(int code) {
    switch (code) {
    case ATOM_ATTN_OK:
        return "ok";
    case ATOM_ATTN_EINVAL:
        return "invalid argument (enum, dim < 1, missing or misaligned pointer, "
               "eps not finite and > 0 in the dtype, radius < -1)";
    case ATOM_ATTN_EODD_HEAD:
        return "ESMFold2 style needs an even head width D";
    case ATOM_ATTN_EWORKSPACE:
        return "workspace missing, misaligned or smaller than atom_attn_workspace_bytes()";
    case ATOM_ATTN_ELAUNCH:
        return "the HIP runtime refused a kernel launch";
    case ATOM_ATTN_ESCRATCH:
        return "these sizes need more scratch than the library's static per-device "
               "buffer holds (atom_attn_block_noalloc; see "
               "atom_attn_noalloc_max_bytes)";
    case ATOM_ATTN_EUNSUPPORTED:
        return "shape outside the supported set (C, S, H*D, M, U multiples of 32 "
               "and <= 512; D one of 16, 32, 64, 128; K <= 256; AF3: V a "
               "multiple of 8 with V*sizeof(dtype) <= 64, H <= 4; "
               "D*(A+39)*sizeof(dtype) < 2^31)";
    default:
        return "unknown status";
    }
}

int atom_attn_workspace_bytes(const atom_attn_dims *dims, int style, int stage,
                              int dtype, size_t *bytes) {
    int rc = check_common(dims, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    if (!bytes)
        return ATOM_ATTN_EINVAL;
    rc = shape_supported(dims, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    *bytes = layout_of(dims, style, stage, dtype).total;
    return ATOM_ATTN_OK;
}

int atom_attn_packed_bytes(const atom_attn_dims *dims, int style, int stage, int dtype,
                           size_t *bytes) {
    int rc = check_common(dims, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    if (!bytes)
        return ATOM_ATTN_EINVAL;
    rc = shape_supported(dims, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    *bytes = (size_t)layout_of(dims, style, stage, dtype).pack_units * 16 * 2;
    return ATOM_ATTN_OK;
}

int atom_attn_pack_params(const atom_attn_dims *dims, int style, int stage, int dtype,
                          const atom_attn_params *par, void *packed, size_t packed_bytes,
                          void *stream) {
    int rc = check_common(dims, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    if (!par || !matrices_present(par, style, stage))
        return ATOM_ATTN_EINVAL;
    rc = shape_supported(dims, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    const Layout L = layout_of(dims, style, stage, dtype);
    if (!packed || !aligned16(packed) || packed_bytes < (size_t)L.pack_units * 32)
        return ATOM_ATTN_EWORKSPACE;
    const int esz = dtype == ATOM_ATTN_BF16 ? 2 : 4;
    const int dt = dtype == ATOM_ATTN_BF16 ? 1 : 0;
    PackedOffsets off;
    MatList mats;
    list_mats(dims, style, stage, esz, par, &off, &mats);
    hipStream_t s = (hipStream_t)stream;
    for (int strips = 0; strips < 2; ++strips) {
        PackArgs pa;
        std::memset(&pa, 0, sizeof(pa));
        pa.njobs = (int)mats.size();
        for (size_t i = 0; i < mats.size(); ++i)
            pa.job[i] = PackJob{mats[i].src, mats[i].ld, mats[i].kd, mats[i].n, *mats[i].off,
                                strips && mats[i].tile ? 1 : 0};
        pa.total = L.pack_units;
        pa.out = (uint4 *)packed + (strips ? L.pack_units : 0);
        if ((rc = timed(KN_PACK, s, [&] { return launch_pack(pa, dt, s); })) != ATOM_ATTN_OK)
            return rc;
    }
    return ATOM_ATTN_OK;
}

int atom_attn_pair_bias_split(const atom_attn_dims *dims, int style, int stage,
                              int dtype, int *split) {
    int rc = check_common(dims, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    if (!split)
        return ATOM_ATTN_EINVAL;
    rc = shape_supported(dims, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    const Dims d{(int)dims->B, (int)dims->A, (int)dims->T, (int)dims->K, (int)dims->C,
                 (int)dims->S, (int)dims->H, (int)dims->D, (int)dims->V, (int)dims->M,
                 (int)dims->U};
    *split = style == ATOM_ATTN_AF3 &&
             prep_hosts_pair_bias(d, dtype == ATOM_ATTN_BF16 ? 1 : 0, STYLE_AF3,
                                  stage == ATOM_ATTN_ENCODER ? STAGE_ENCODER : STAGE_DECODER);
    return ATOM_ATTN_OK;
}

int atom_attn_encoder(const atom_attn_dims *dims, int style, int dtype,
                      const atom_attn_inputs *in, const atom_attn_params *par,
                      double eps, int64_t radius, atom_attn_outputs *out,
                      void *workspace, size_t workspace_bytes, void *stream) {
    return run_block(dims, style, ATOM_ATTN_ENCODER, dtype, in, par, eps, radius,
                     out, workspace, workspace_bytes, stream);
}

int atom_attn_decoder(const atom_attn_dims *dims, int style, int dtype,
                      const atom_attn_inputs *in, const atom_attn_params *par,
                      double eps, int64_t radius, atom_attn_outputs *out,
                      void *workspace, size_t workspace_bytes, void *stream) {
    return run_block(dims, style, ATOM_ATTN_DECODER, dtype, in, par, eps, radius,
                     out, workspace, workspace_bytes, stream);
}

int atom_attn_masks(const atom_attn_dims *dims, const atom_attn_inputs *in,
                    int64_t radius, uint8_t *usable, uint8_t *allowed,
                    int32_t *token_count, void *stream) {
    if (!dims || dims->B < 1 || dims->A < 1 || dims->T < 1 || dims->K < 1 || !in ||
        radius < -1 || !in->valid || !in->token_valid || !in->window_mask ||
        !in->atom_to_token || !in->key_index || (!usable && !allowed && !token_count))
        return ATOM_ATTN_EINVAL;
    if (dims->B * dims->A * dims->K > ((int64_t)1 << 40) ||
        dims->A > ((int64_t)1 << 30) || dims->B * dims->T > ((int64_t)1 << 31) - 1)
        return ATOM_ATTN_EUNSUPPORTED;
    const Dims d{(int)dims->B, (int)dims->A, (int)dims->T, (int)dims->K, 1, 1, 1, 1, 1, 1, 1};
    hipStream_t s = (hipStream_t)stream;
    return timed(KN_MASKS, s, [&] {
        return launch_masks(d, in->valid, in->token_valid, in->window_mask,
                            in->atom_to_token, in->key_index, radius, usable,
                            allowed, token_count, s);
    });
}

int atom_attn_slot_workspace_bytes(const atom_attn_dims *dims, int dtype,
                                   size_t *bytes) {
    if (!dims || dims->B < 1 || dims->A < 1 || dims->H < 1 || dims->D < 1 || !bytes ||
        (dtype != ATOM_ATTN_F32 && dtype != ATOM_ATTN_BF16))
        return ATOM_ATTN_EINVAL;
    const size_t esz = dtype == ATOM_ATTN_BF16 ? 2 : 4;
    // transposed v, then the queue of wide query blocks
    *bytes = up256((size_t)(dims->B * dims->H * dims->D) * vt_pitch((int)dims->A) * esz) +
             up256(4 * ((size_t)dims->B * ((dims->A + 15) / 16) + 1));
    return ATOM_ATTN_OK;
}

int atom_attn_slot_attention(const atom_attn_dims *dims, int style, int dtype,
                             double eps, int64_t radius, const uint8_t *usable,
                             const void *q, const void *k, const void *v,
                             const int64_t *key_index,
                             const uint8_t *window_mask, const void *pair,
                             const void *pair_scale, const void *w_pair,
                             void *attention, void *o, void *workspace,
                             size_t workspace_bytes, void *stream) {
    if (!dims || dims->B < 1 || dims->A < 1 || dims->K < 1 || dims->H < 1 ||
        dims->D < 1 || (style == ATOM_ATTN_AF3 && dims->V < 1))
        return ATOM_ATTN_EINVAL;
    if (style != ATOM_ATTN_AF3 && style != ATOM_ATTN_ESMFOLD2)
        return ATOM_ATTN_EINVAL;
    if (dtype != ATOM_ATTN_F32 && dtype != ATOM_ATTN_BF16)
        return ATOM_ATTN_EINVAL;
    if (!eps_valid(eps, dtype) || radius < -1)
        return ATOM_ATTN_EINVAL;
    if (!usable || !key_index || !window_mask)
        return ATOM_ATTN_EINVAL;
    const void *need[] = {q, k, v, attention, o};
    for (const void *p : need)
        if (!p || !aligned16(p))
            return ATOM_ATTN_EINVAL;
    if (style == ATOM_ATTN_AF3 && (!pair || !pair_scale || !w_pair || !aligned16(pair)))
        return ATOM_ATTN_EINVAL;
    if (style == ATOM_ATTN_ESMFOLD2 && dims->D % 2 != 0)
        return ATOM_ATTN_EODD_HEAD;
    const int64_t HD = dims->H * dims->D;
    if (HD % 32 != 0 || HD > 512)
        return ATOM_ATTN_EUNSUPPORTED;
    const Dims d{(int)dims->B, (int)dims->A, 1, (int)dims->K, 32, 32, (int)dims->H,
                 (int)dims->D, style == ATOM_ATTN_AF3 ? (int)dims->V : 8, 32, 32};
    const int dt = dtype == ATOM_ATTN_BF16 ? 1 : 0;
    const int st = style == ATOM_ATTN_AF3 ? STYLE_AF3 : STYLE_ESM;
    if (!slot_supported(d, dt, st) || dims->B * dims->A > ((int64_t)1 << 30) ||
        dims->B * dims->H * dims->A * dims->K > ((int64_t)1 << 31) - 1 ||
        !vt_offsets_fit(dims->A, dims->D, dt ? 2 : 4))
        return ATOM_ATTN_EUNSUPPORTED;
    size_t need_ws = 0;
    atom_attn_slot_workspace_bytes(dims, dtype, &need_ws);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need_ws)
        return ATOM_ATTN_EWORKSPACE;
    SlotArgs sa;
    std::memset(&sa, 0, sizeof(sa)); // pbias null: the pair bias comes from the pair rows
    sa.B = d.B; sa.A = d.A; sa.K = d.K; sa.H = d.H; sa.D = d.D; sa.V = d.V;
    sa.eps = (float)eps;
    sa.inv_sqrt_d = (float)(1.0 / std::sqrt((double)d.D));
    sa.radius = radius;
    sa.usable = usable; sa.window_mask = window_mask; sa.key_index = key_index;
    sa.q = q; sa.k = k; sa.v = workspace;
    sa.pair = pair; sa.pair_scale = pair_scale; sa.w_pair = w_pair;
    sa.attention = attention; sa.o = o;
    const size_t vt_bytes = up256((size_t)(dims->B * dims->H * dims->D) * vt_pitch((int)dims->A) *
                                  (dt ? 2 : 4));
    sa.wide = (int *)((char *)workspace + vt_bytes);
    sa.vrows = v; // the caller's rows serve the gather path
    hipStream_t s = (hipStream_t)stream;
    if (launch_vt(v, usable, workspace, d.B, d.A, (int)HD, dt, sa.wide, s) != hipSuccess)
        return ATOM_ATTN_ELAUNCH;
    const int rc = timed(KN_SLOT, s, [&] { return launch_slot(sa, dt, st, s); });
    if (rc != ATOM_ATTN_OK)
        return rc;
    return timed(KN_SLOT_GATHER, s, [&] { return launch_slot_gather(sa, dt, st, s); });
}

int atom_attn_profile_enable(int on) {
    g_prof.on = on != 0;
    return ATOM_ATTN_OK;
}

int atom_attn_profile_read(const char **names, double *total_ms, int64_t *launches,
                           int max) {
    double tot[32] = {0};
    int64_t cnt[32] = {0};
    for (auto &r : g_prof.recs) {
        if (hipEventSynchronize(r.stop) != hipSuccess)
            return ATOM_ATTN_ELAUNCH;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
            return ATOM_ATTN_ELAUNCH;
        tot[r.kernel] += ms;
        cnt[r.kernel] += 1;
        g_prof.pool.push_back(r.start);
        g_prof.pool.push_back(r.stop);
    }
    g_prof.recs.clear();
    int w = 0;
    for (int i = 0; i < g_prof.nnames && w < max; ++i) {
        if (cnt[i] == 0)
            continue;
        if (names)
            names[w] = g_prof.names[i];
        if (total_ms)
            total_ms[w] = tot[i];
        if (launches)
            launches[w] = cnt[i];
        ++w;
    }
    return w;
}

} // extern "C"
