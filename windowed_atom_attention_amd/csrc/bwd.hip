// bwd.hip -- the C ABI of the backward pass (declared in include/atom_attn.h):
// atom_attn_backward, the gradients of every float input and parameter of
// the block, and atom_attn_slot_attention_backward, the slot step alone.
// Host code only: the forward intermediates the chain rule needs are
// recomputed in fp32 from the inputs, then the chain rule runs from the
// outputs back to the inputs, every step in the kernels of bwd_dense.hip
// and bwd_slot.hip.
//
// Pages: "windowed_atom_attention" (Required behavior: the block, and the
// repeated-selection rule for gradients), "AlphaFold 3 Atom Attention
// Encoder" and "ESMFold 2 Atom Attention Encoder" (Required behavior; their
// Starter code grades gradients).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <unordered_map>

#include "../../include/atom_attn.h"
#include "bwd.hpp"
#include "kernels.hpp"

using namespace waa;
using namespace waa::bwd;

namespace {

struct Arena {
    char *base;
    size_t off = 0;
    template <typename T> T *get(size_t n) {
        off = (off + 255) & ~(size_t)255;
        T *p = base ? reinterpret_cast<T *>(base + off) : nullptr;
        off += std::max<size_t>(n, 1) * sizeof(T);
        return p;
    }
};

bool eps_ok(double eps) {
    return eps > 0.0 && std::isfinite(eps) && (float)eps > 0.0f && std::isfinite((float)eps);
}

// Shapes the backward kernels handle (the dense kernels take any sizes).
int bwd_shape_ok(const atom_attn_dims *d, int style) {
    if (!slot_bwd_supported((int)d->K, (int)d->H, (int)d->D, (int)d->V,
                            style == ATOM_ATTN_AF3 ? STYLE_AF3 : STYLE_ESM))
        return ATOM_ATTN_EUNSUPPORTED;
    const int64_t N = d->B * d->A;
    if (N >= ((int64_t)1 << 30) || N * d->K * std::max<int64_t>(d->H, d->V) >= ((int64_t)1 << 31) ||
        d->B * d->T >= ((int64_t)1 << 30))
        return ATOM_ATTN_EUNSUPPORTED;
    const int64_t widths[] = {d->C, d->S, d->M, d->U};
    for (int64_t x : widths)
        if (x > 4096)
            return ATOM_ATTN_EUNSUPPORTED;
    // every intermediate (rows x widest row, 6C for the ESMFold2 modulations)
    // below 2^34 elements: the grouped launches count workgroups and tiles
    // of up to eight such jobs in 32 bits
    const int64_t wmax = std::max<int64_t>({6 * d->C, d->S, d->M, d->U, d->H * d->D});
    if (N * wmax > ((int64_t)1 << 34))
        return ATOM_ATTN_EUNSUPPORTED;
    return ATOM_ATTN_OK;
}

// Every buffer of one backward call, carved from the workspace.
struct Bufs {
    // fp32 parameters
    float *cs, *ws, *bs, *wsh, *wrg, *brg, *wmod, *wq, *bq, *wk, *wv, *ps, *wp, *wvg, *wao;
    float *ffg, *ffu, *ffo, *wpool, *wtok, *rs, *rb, *wro;
    // masks
    uint8_t *usable, *allowed;
    int32_t *tcount;
    // recomputed forward
    float *tok, *tokproj, *x0, *c, *ch, *rc, *cj[3], *sig[3], *mu[3], *gr[2], *mods, *sc;
    float *xh0, *r0, *qin, *kvin, *qraw, *kraw, *rcos, *rsin, *q, *k, *v, *g, *P, *o;
    int32_t *kid;
    float *og, *uu, *x1, *xh1, *r1, *z, *fa, *fb, *hh, *tr, *hid, *proj, *xhh, *rh, *lnh;
    // backward
    float *dh, *dx2, *dtr, *dhh, *da, *dbb, *dz, *dx1, *gt, *du, *dog, *dO, *dGp;
    float *dS, *dq, *dk, *dv, *dqin, *dkvin, *dx0, *dzs[3], *dzg[2], *dcj[3], *dch, *dc, *dmods,
        *ds, *dpu, *dln, *dtp, *dP, *pwp, *part, *part2, *Pk;
    int32_t *tkey, *tcnt, *toff, *tlist, *cnt, *off, *list, *inv, *wide;
};

void carve(Arena &ar, const atom_attn_dims *d, int style, int stage, Bufs &b) {
    std::memset(&b, 0, sizeof(b));
    const size_t B = d->B, A = d->A, T = d->T, K = d->K, C = d->C, S = d->S, H = d->H,
                 D = d->D, V = d->V, M = d->M, U = d->U;
    const size_t N = B * A, E = N * K, HD = H * D, BT = B * T;
    const bool af3 = style == ATOM_ATTN_AF3, dec = stage == ATOM_ATTN_DECODER;
    auto f = [&](size_t n) { return ar.get<float>(n); };
    if (af3) {
        b.cs = f(3 * S); b.ws = f(3 * S * C); b.bs = f(3 * C); b.wsh = f(3 * S * C);
        b.wrg = f(2 * S * C); b.brg = f(2 * C); b.bq = f(HD); b.ps = f(V); b.wp = f(V * H);
    } else {
        b.wmod = f(S * 6 * C);
    }
    b.wq = f(C * HD); b.wk = f(C * HD); b.wv = f(C * HD); b.wvg = f(C * HD); b.wao = f(HD * C);
    b.ffg = f(C * M); b.ffu = f(C * M); b.ffo = f(M * C);
    if (dec) {
        b.wtok = f(U * C); b.rs = f(C); b.rb = f(C); b.wro = f(C * 3);
    } else {
        b.wpool = f(C * U);
    }
    b.usable = ar.get<uint8_t>(N);
    b.allowed = ar.get<uint8_t>(E);
    b.tcount = ar.get<int32_t>(BT);
    if (dec) {
        b.tok = f(BT * U); b.tokproj = f(BT * C);
    }
    b.x0 = f(N * C); b.c = f(N * S); b.xh0 = f(N * C); b.r0 = f(N); b.qin = f(N * C);
    if (af3) {
        b.ch = f(N * S); b.rc = f(N);
        for (int j = 0; j < 3; ++j) b.cj[j] = f(N * S);
        for (int j = 0; j < 3; ++j) { b.sig[j] = f(N * C); b.mu[j] = f(N * C); }
        for (int j = 0; j < 2; ++j) b.gr[j] = f(N * C);
        b.kvin = f(N * C);
    } else {
        b.mods = f(N * 6 * C); b.sc = f(N * S); b.kvin = b.qin;
        b.qraw = f(N * HD); b.kraw = f(N * HD); b.rcos = f(N * D); b.rsin = f(N * D);
    }
    b.q = f(N * HD); b.k = f(N * HD); b.v = f(N * HD); b.g = f(N * HD);
    b.P = f(E * H); b.o = f(N * HD); b.kid = ar.get<int32_t>(E);
    b.og = f(N * HD); b.uu = f(N * C); b.x1 = f(N * C); b.xh1 = f(N * C); b.r1 = f(N);
    b.z = f(N * C); b.fa = f(N * M); b.fb = f(N * M); b.hh = f(N * M); b.tr = f(N * C);
    b.hid = f(N * C);
    if (dec) {
        b.xhh = f(N * C); b.rh = f(N); b.lnh = f(N * C);
    } else {
        b.proj = f(N * U);
    }
    b.dh = f(N * C); b.dx2 = f(N * C); b.dtr = f(N * C);
    b.dhh = f(N * M); b.da = f(N * M); b.dbb = f(N * M); b.dz = f(N * C); b.dx1 = f(N * C);
    b.gt = f(N * C); b.du = f(N * C); b.dog = f(N * HD); b.dO = f(N * HD);
    b.dGp = f(N * HD); b.dS = f(E * H); b.dq = f(N * HD); b.dk = f(N * HD); b.dv = f(N * HD);
    b.dqin = f(N * C); b.dkvin = f(N * C); b.dx0 = f(N * C); b.dc = f(N * S);
    if (af3) {
        for (int j = 0; j < 3; ++j) b.dzs[j] = f(N * C);
        for (int j = 0; j < 2; ++j) b.dzg[j] = f(N * C);
        for (int j = 0; j < 3; ++j) b.dcj[j] = f(N * S);
        b.dch = f(N * S);
    } else {
        b.dmods = f(N * 6 * C); b.ds = f(N * S);
    }
    if (dec) {
        b.dpu = f(N * 3); b.dln = f(N * C); b.dtp = f(BT * C);
        b.tkey = ar.get<int32_t>(N); b.tcnt = ar.get<int32_t>(reverse_index_count_ints(BT));
        b.toff = ar.get<int32_t>(BT + 1); b.tlist = ar.get<int32_t>(N);
    } else {
        b.dP = f(N * U);
    }
    b.cnt = ar.get<int32_t>(reverse_index_count_ints(N)); b.off = ar.get<int32_t>(N + 1);
    b.list = ar.get<int32_t>(E); b.inv = ar.get<int32_t>(E); b.Pk = f(E * H);
    b.pwp = f(slot_bwd_partial_floats((int64_t)B, (int64_t)A, (int)V, (int)H));
    b.wide = ar.get<int32_t>(slot_bwd_queue_ints((int64_t)B, (int64_t)A));
    b.part = f(kGemmPartialFloats);
    b.part2 = f(kGemmPartialFloats);
}

// A second stream per device for the parameter gradients: every product
// or column sum whose result is a parameter gradient is a leaf of the
// chain rule (nothing downstream reads it), so it can run beside the main
// chain. Default priority; fork and join through events.
struct Side {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex enqueue; // one backward call at a time enqueues on a device
};
Side *side_stream() {
    static std::mutex mu;
    static std::unordered_map<int, Side *> per_dev;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return nullptr;
    std::lock_guard<std::mutex> lk(mu);
    Side *&x = per_dev[dev];
    if (!x) {
        Side *n = new Side();
        if (hipStreamCreateWithFlags(&n->s, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&n->fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&n->join, hipEventDisableTiming) != hipSuccess)
            return nullptr; // (leaked on failure; the call then stays on one stream)
        x = n;
    }
    return x;
}

// Sequenced launches that stop at the first failure.
struct Run {
    hipStream_t s;
    Scratch sc;
    Side *side = nullptr; // null: leaves run on the main stream
    Scratch sc2{};
    hipError_t err = hipSuccess;
    // parameter-gradient leaves queued since the last fork; they go out as
    // grouped launches (leaf_group) when the next fork or the join comes.
    // Their inputs stay valid until the join (the main chain never rewrites
    // a buffer a leaf reads), so the deferral changes no value.
    LeafJob pending[64];
    int npend = 0;
    void flush() {
        for (int i = 0; i < npend && err == hipSuccess; i += kLeafJobs)
            ok(leaf_group(pending + i, std::min(kLeafJobs, npend - i), side ? sc2 : sc,
                          side ? side->s : s));
        npend = 0;
    }
    // make the side stream wait for everything enqueued on the main stream
    void fork() {
        flush();
        if (side && err == hipSuccess) {
            ok(hipEventRecord(side->fork, s));
            ok(hipStreamWaitEvent(side->s, side->fork, 0));
        }
    }
    void join() {
        flush();
        if (side) {
            ok(hipEventRecord(side->join, side->s));
            ok(hipStreamWaitEvent(s, side->join, 0));
        }
    }
    void queue(const LeafJob &x) {
        if (npend == 64)
            flush();
        pending[npend++] = x;
    }
    // a parameter-gradient product / column sum (after a fork)
    void leaf_mm(int M, int N, int K, Mat A, Mat B, float *C, int64_t ldc) {
        if (err == hipSuccess && C)
            queue(LeafJob{0, M, N, K, A, B, C, ldc});
    }
    void leaf_cs(int rows, int W, const float *X, int64_t ldx, const float *Y, int64_t ldy,
                 float *out) {
        if (err == hipSuccess && out)
            queue(LeafJob{1, 1, W, rows, mat(X, ldx), Mat{Y, ldy, 1}, out, W});
    }
    void ok(hipError_t e) {
        if (err == hipSuccess && e != hipSuccess)
            err = e;
    }
    // C (+)= A @ B, A [M,K], B [K,N]
    void mm(int M, int N, int K, Mat A, Mat B, float *C, int64_t ldc, float beta = 0.0f,
            const float *bias = nullptr) {
        if (err == hipSuccess)
            ok(gemm(M, N, K, A, B, View{C, ldc}, beta, bias, sc, s));
    }
    void e(EwOp op, int rows, int W, float *o, int64_t ldo, const float *a, int64_t lda,
           const float *b = nullptr, int64_t ldb = 0, const float *c = nullptr, int64_t ldc = 0,
           const float *vec = nullptr, const uint8_t *mask = nullptr, int acc = 0) {
        if (err == hipSuccess)
            ok(ew(op, rows, W, View{o, ldo}, view(a, lda), view(b, ldb), view(c, ldc), vec, mask,
                  acc, s));
    }
    // independent products / elementwise jobs in one launch each
    void mmg(std::initializer_list<GemmJob> jobs) { mmg(jobs.begin(), (int)jobs.size()); }
    void mmg(const GemmJob *jobs, int n) {
        if (err == hipSuccess)
            ok(gemm_group(jobs, n, s));
    }
    void eg(std::initializer_list<EwJob> jobs) { eg(jobs.begin(), (int)jobs.size()); }
    void eg(const EwJob *jobs, int n) {
        if (err == hipSuccess && n > 0)
            ok(ew_group(jobs, n, s));
    }
    void cs(int rows, int W, const float *X, int64_t ldx, const float *Y, int64_t ldy, float *out) {
        if (err == hipSuccess && out)
            ok(colsum(rows, W, view(X, ldx), view(Y, ldy), out, 0.0f, sc, s));
    }
    void norm(int mode, int rows, int W, float eps, const float *x, float *xh, float *r) {
        if (err == hipSuccess)
            ok(norm_rows(mode, rows, W, eps, view(x, W), view(xh, W), r, s));
    }
    void norm_bwd(int mode, int rows, int W, const float *xh, const float *r, const float *g,
                  float *o, int acc) {
        if (err == hipSuccess)
            ok(norm_rows_bwd(mode, rows, W, view(xh, W), r, view(g, W), view(o, W), acc, s));
    }
    void cvt(const void *src, int dtype, int64_t n, float *dst) {
        if (err == hipSuccess && src)
            ok(to_f32(src, dtype, 1, (int)n, n, dst, nullptr, s));
    }
};

// One product job: C (+)= sum of the segments' A B (+ bias), then epi.
GemmJob gj(int M, int N, float *C, int64_t ldc, std::initializer_list<GemmSeg> segs,
           const float *bias = nullptr, int epi = GEMM_NONE) {
    GemmJob j{};
    j.M = M;
    j.N = N;
    j.C = View{C, ldc};
    j.beta = 0.0f;
    j.bias = bias;
    j.epi = epi;
    for (const GemmSeg &x : segs)
        j.seg[j.nseg++] = x;
    return j;
}
GemmSeg sg(int K, Mat A, Mat B) { return GemmSeg{A, B, K}; }
// One elementwise job (operands as for Run::e; d and vec2/vec3 set apart).
EwJob ej(EwOp op, int rows, int W, float *o, int64_t ldo, const float *a, int64_t lda,
         const float *b = nullptr, int64_t ldb = 0, const float *c = nullptr, int64_t ldc = 0,
         const float *vec = nullptr, const uint8_t *mask = nullptr, int acc = 0) {
    return EwJob{op, rows, W, View{o, ldo}, view(a, lda), view(b, ldb), view(c, ldc),
                 View{nullptr, 0}, vec, nullptr, nullptr, mask, acc};
}

int run_backward(const atom_attn_dims *d, int style, int stage, int dtype,
                 const atom_attn_inputs *in, const atom_attn_params *par, float eps,
                 int64_t radius, const atom_attn_grad_outputs *gout, atom_attn_input_grads *gin,
                 atom_attn_param_grads *gpar, void *workspace, hipStream_t s) {
    Arena ar{(char *)workspace};
    Bufs b;
    carve(ar, d, style, stage, b);
    const int B = (int)d->B, A = (int)d->A, T = (int)d->T, K = (int)d->K, C = (int)d->C,
              S = (int)d->S, H = (int)d->H, D = (int)d->D, V = (int)d->V, M = (int)d->M,
              U = (int)d->U;
    const int N = B * A, HD = H * D, BT = B * T;
    const bool af3 = style == ATOM_ATTN_AF3, dec = stage == ATOM_ATTN_DECODER;
    const int nm = af3 ? 0 : 1; // row normalisation: LayerNorm (AF3) / RMS (ESMFold2)
    const int C6 = 6 * C;
    Run r{s, Scratch{b.part, kGemmPartialFloats}};
    Side *side = side_stream();
    std::unique_lock<std::mutex> lk;
    if (side) {
        lk = std::unique_lock<std::mutex>(side->enqueue);
        r.side = side;
        r.sc2 = Scratch{b.part2, kGemmPartialFloats};
    }

    // ---------------------------------------------------------- recompute
    ProfSpan sp = prof_begin(KN_BWD_RECOMPUTE, s);
    // parameters in fp32: used in place when stored as fp32, else widened
    auto prm = [&](const void *src, int64_t n, float *&dst) {
        if (!src)
            return;
        if (dtype == ATOM_ATTN_F32)
            dst = const_cast<float *>(static_cast<const float *>(src));
        else
            r.cvt(src, dtype, n, dst);
    };
    if (af3) {
        prm(par->cond_scale, 3 * S, b.cs);
        prm(par->w_scale, 3 * (int64_t)S * C, b.ws);
        prm(par->b_scale, 3 * C, b.bs);
        prm(par->w_shift, 3 * (int64_t)S * C, b.wsh);
        prm(par->w_residual_gate, 2 * (int64_t)S * C, b.wrg);
        prm(par->b_residual_gate, 2 * C, b.brg);
        prm(par->b_q, HD, b.bq);
        prm(par->pair_scale, V, b.ps);
        prm(par->w_pair, (int64_t)V * H, b.wp);
    } else {
        prm(par->w_mod, (int64_t)S * C6, b.wmod);
    }
    prm(par->w_q, (int64_t)C * HD, b.wq);
    prm(par->w_k, (int64_t)C * HD, b.wk);
    prm(par->w_v, (int64_t)C * HD, b.wv);
    prm(par->w_value_gate, (int64_t)C * HD, b.wvg);
    prm(par->w_attention_out, (int64_t)HD * C, b.wao);
    prm(par->w_ff_gate, (int64_t)C * M, b.ffg);
    prm(par->w_ff_up, (int64_t)C * M, b.ffu);
    prm(par->w_ff_out, (int64_t)M * C, b.ffo);
    if (dec) {
        prm(par->w_token, (int64_t)U * C, b.wtok);
        prm(par->readout_scale, C, b.rs);
        if (!af3)
            prm(par->readout_bias, C, b.rb);
        prm(par->w_readout, (int64_t)C * 3, b.wro);
    } else {
        prm(par->w_pool, (int64_t)C * U, b.wpool);
    }
    const Dims dd{B, A, T, K, C, S, H, D, V, M, U};
    r.ok(launch_masks(dd, in->valid, in->token_valid, in->window_mask, in->atom_to_token,
                      in->key_index, radius, b.usable, b.allowed, b.tcount, s));
    if (dec) {
        // token rows of invalid tokens never reach a usable atom: zeros
        if (r.err == hipSuccess)
            r.ok(to_f32(in->token, dtype, BT, U, U, b.tok, in->token_valid, s));
        r.mm(BT, C, U, mat(b.tok, U), mat(b.wtok, C), b.tokproj, C);
    }
    if (r.err == hipSuccess)
        r.ok(sanitize(B, A, T, C, S, dtype, in->atom, in->condition, b.usable, in->atom_to_token,
                      dec ? b.tokproj : nullptr, b.x0, b.c, s));
    // conditioning
    if (af3) {
        r.norm(0, N, S, eps, b.c, b.ch, b.rc);
        r.eg({ej(EW_MUL_VEC, N, S, b.cj[0], S, b.ch, S, nullptr, 0, nullptr, 0, b.cs),
              ej(EW_MUL_VEC, N, S, b.cj[1], S, b.ch, S, nullptr, 0, nullptr, 0, b.cs + S),
              ej(EW_MUL_VEC, N, S, b.cj[2], S, b.ch, S, nullptr, 0, nullptr, 0, b.cs + 2 * S)});
        // the eight conditioning products (sigmoid gates with their biases)
        GemmJob js[kGroupJobs];
        int nj = 0;
        for (int j = 0; j < 3; ++j) {
            js[nj++] = gj(N, C, b.sig[j], C, {sg(S, mat(b.cj[j], S), mat(b.ws + (size_t)j * S * C, C))},
                          b.bs + j * C, GEMM_SIGMOID);
            js[nj++] = gj(N, C, b.mu[j], C, {sg(S, mat(b.cj[j], S), mat(b.wsh + (size_t)j * S * C, C))});
        }
        for (int j = 0; j < 2; ++j)
            js[nj++] = gj(N, C, b.gr[j], C, {sg(S, mat(b.c, S), mat(b.wrg + (size_t)j * S * C, C))},
                          b.brg + j * C, GEMM_SIGMOID);
        r.mmg(js, nj);
    } else {
        r.e(EW_SILU, N, S, b.sc, S, b.c, S);
        r.mm(N, C6, S, mat(b.sc, S), mat(b.wmod, C6), b.mods, C6);
    }
    const float *gA = af3 ? b.gr[0] : b.mods + 2 * C;
    const float *gT = af3 ? b.gr[1] : b.mods + 5 * C;
    const int64_t ldg = af3 ? C : C6;
    // modulated norms
    r.norm(nm, N, C, eps, b.x0, b.xh0, b.r0);
    if (af3)
        r.eg({ej(EW_AFFINE, N, C, b.qin, C, b.xh0, C, b.sig[0], C, b.mu[0], C),
              ej(EW_AFFINE, N, C, b.kvin, C, b.xh0, C, b.sig[1], C, b.mu[1], C)});
    else
        r.e(EW_AFFINE1, N, C, b.qin, C, b.xh0, C, b.mods + C, C6, b.mods, C6);
    // projections (the value gate's sigmoid in the product's epilogue)
    float *qdst = af3 ? b.q : b.qraw;
    float *kdst = af3 ? b.k : b.kraw;
    r.mmg({gj(N, HD, qdst, HD, {sg(C, mat(b.qin, C), mat(b.wq, HD))}, af3 ? b.bq : nullptr),
           gj(N, HD, kdst, HD, {sg(C, mat(b.kvin, C), mat(b.wk, HD))}),
           gj(N, HD, b.v, HD, {sg(C, mat(b.kvin, C), mat(b.wv, HD))}),
           gj(N, HD, b.g, HD, {sg(C, mat(b.qin, C), mat(b.wvg, HD))}, nullptr, GEMM_SIGMOID)});
    float *dcos = gin ? gin->rope_cos : nullptr, *dsin = gin ? gin->rope_sin : nullptr;
    const float *cs_f = nullptr, *sn_f = nullptr;
    if (!af3) {
        float *ct = b.rcos, *st = b.rsin; // rotary tables in fp32
        if (r.err == hipSuccess) {
            r.ok(to_f32(in->rope_cos, dtype, N, D, D, ct, nullptr, s));
            r.ok(to_f32(in->rope_sin, dtype, N, D, D, st, nullptr, s));
        }
        cs_f = ct;
        sn_f = st;
        if (r.err == hipSuccess)
            r.ok(head_rope(N, H, D, eps, b.qraw, b.kraw, ct, st, b.q, b.k, s));
    }
    prof_end(sp, s);
    // slot attention with its weights kept
    SlotBwdArgs sa{};
    sa.B = B; sa.A = A; sa.K = K; sa.H = H; sa.D = D; sa.V = V;
    sa.eps = eps; sa.radius = radius; sa.pair_dtype = dtype;
    sa.usable = b.usable; sa.window_mask = in->window_mask; sa.key_index = in->key_index;
    sa.q = b.q; sa.k = b.k; sa.v = b.v; sa.pair = af3 ? in->pair : nullptr;
    sa.ps = b.ps; sa.wp = b.wp; sa.P = b.P; sa.o = b.o; sa.kid = b.kid;
    sa.d_att = gout->attention; sa.d_o = b.dO; sa.dS = b.dS;
    sa.dq = b.dq; sa.dk = b.dk; sa.dv = b.dv; sa.d_pair = (af3 && gin) ? gin->pair : nullptr;
    sa.pw_partial = b.pwp; sa.count = b.cnt; sa.offset = b.off; sa.list = b.list;
    sa.inv = b.inv; sa.Pk = b.Pk; sa.wide = b.wide;
    sa.sc = r.sc;
    if (r.err == hipSuccess) {
        sp = prof_begin(KN_BWD_SLOT_FWD, s);
        r.ok(slot_fwd(sa, af3 ? STYLE_AF3 : STYLE_ESM, s));
        prof_end(sp, s);
    }
    sp = prof_begin(KN_BWD_RECOMPUTE, s);
    r.e(EW_MUL, N, HD, b.og, HD, b.o, HD, b.g, HD);
    r.mm(N, C, HD, mat(b.og, HD), mat(b.wao, C), b.uu, C);
    r.e(EW_RESID, N, C, b.x1, C, b.x0, C, gA, ldg, b.uu, C);
    r.norm(nm, N, C, eps, b.x1, b.xh1, b.r1);
    if (af3)
        r.e(EW_AFFINE, N, C, b.z, C, b.xh1, C, b.sig[2], C, b.mu[2], C);
    else
        r.e(EW_AFFINE1, N, C, b.z, C, b.xh1, C, b.mods + 4 * C, C6, b.mods + 3 * C, C6);
    r.mmg({gj(N, M, b.fa, M, {sg(C, mat(b.z, C), mat(b.ffg, M))}),
           gj(N, M, b.fb, M, {sg(C, mat(b.z, C), mat(b.ffu, M))})});
    r.e(EW_SWIGLU, N, M, b.hh, M, b.fa, M, b.fb, M);
    r.mm(N, C, M, mat(b.hh, M), mat(b.ffo, C), b.tr, C);
    r.e(EW_RESID_MASK, N, C, b.hid, C, b.x1, C, gT, ldg, b.tr, C, nullptr, b.usable);
    if (dec) {
        r.norm(0, N, C, eps, b.hid, b.xhh, b.rh);
        r.e(EW_MUL_VEC, N, C, b.lnh, C, b.xhh, C, nullptr, 0, nullptr, 0, b.rs);
        if (!af3)
            r.e(EW_ADD_VEC, N, C, b.lnh, C, b.lnh, C, nullptr, 0, nullptr, 0, b.rb);
    } else {
        r.mm(N, U, C, mat(b.hid, C), mat(b.wpool, U), b.proj, U);
    }
    prof_end(sp, s);

    // ------------------------------------------------------------ chain rule
    sp = prof_begin(KN_BWD_CHAIN, s);
    if (gout->hidden)
        r.e(EW_COPY, N, C, b.dh, C, gout->hidden, C);
    else
        r.e(EW_ZERO, N, C, b.dh, C, nullptr, 0);
    if (!dec) {
        float *dwpool = gpar ? gpar->w_pool : nullptr;
        if (gout->token_output) {
            if (r.err == hipSuccess)
                r.ok(pool_bwd(B, A, T, U, b.usable, in->atom_to_token, b.tcount,
                              gout->token_output, b.proj, b.dP, s));
            r.fork();
            r.leaf_mm(C, U, N, mat_t(b.hid, C), mat(b.dP, U), dwpool, U);
            r.mm(N, C, U, mat(b.dP, U), mat_t(b.wpool, U), b.dh, C, 1.0f);
        } else if (dwpool) {
            r.e(EW_ZERO, C, U, dwpool, U, nullptr, 0);
        }
    } else {
        float *dwro = gpar ? gpar->w_readout : nullptr;
        float *drs = gpar ? gpar->readout_scale : nullptr;
        float *drb = (gpar && !af3) ? gpar->readout_bias : nullptr;
        if (gout->position_update) {
            r.e(EW_MASK, N, 3, b.dpu, 3, gout->position_update, 3, nullptr, 0, nullptr, 0, nullptr,
                b.usable);
            r.mm(N, C, 3, mat(b.dpu, 3), mat_t(b.wro, 3), b.dln, C);
            r.fork();
            r.leaf_mm(C, 3, N, mat_t(b.lnh, C), mat(b.dpu, 3), dwro, 3);
            r.leaf_cs(N, C, b.dln, C, b.xhh, C, drs);
            r.leaf_cs(N, C, b.dln, C, nullptr, 0, drb);
            r.e(EW_MUL_VEC, N, C, b.gt, C, b.dln, C, nullptr, 0, nullptr, 0, b.rs);
            r.norm_bwd(0, N, C, b.xhh, b.rh, b.gt, b.dh, 1);
        } else {
            if (dwro)
                r.e(EW_ZERO, C, 3, dwro, 3, nullptr, 0);
            if (drs)
                r.e(EW_ZERO, 1, C, drs, C, nullptr, 0);
            if (drb)
                r.e(EW_ZERO, 1, C, drb, C, nullptr, 0);
        }
    }
    // hidden = usable ? x1 + gT * tr : 0
    // (the gate's gradient dh * tr goes straight into its pre-activation
    // gradient: AF3 through the sigmoid, ESMFold2 into the modulation row)
    r.eg({ej(EW_MASK, N, C, b.dx2, C, b.dh, C, nullptr, 0, nullptr, 0, nullptr, b.usable),
          ej(EW_MUL, N, C, b.dtr, C, b.dh, C, gT, ldg, nullptr, 0, nullptr, b.usable),
          af3 ? ej(EW_DGATE, N, C, b.dzg[1], C, b.dh, C, b.tr, C, b.gr[1], C, nullptr, b.usable)
              : ej(EW_MUL, N, C, b.dmods + 5 * C, C6, b.dh, C, b.tr, C, nullptr, 0, nullptr,
                   b.usable)});
    // transition
    r.fork();
    r.leaf_mm(M, C, N, mat_t(b.hh, M), mat(b.dtr, C), gpar ? gpar->w_ff_out : nullptr, C);
    r.mm(N, M, C, mat(b.dtr, C), mat_t(b.ffo, C), b.dhh, M);
    r.eg({ej(EW_DSWIGLU_A, N, M, b.da, M, b.dhh, M, b.fa, M, b.fb, M),
          ej(EW_DSWIGLU_B, N, M, b.dbb, M, b.dhh, M, b.fa, M)});
    r.fork();
    r.leaf_mm(C, M, N, mat_t(b.z, C), mat(b.da, M), gpar ? gpar->w_ff_gate : nullptr, M);
    r.leaf_mm(C, M, N, mat_t(b.z, C), mat(b.dbb, M), gpar ? gpar->w_ff_up : nullptr, M);
    r.mmg({gj(N, C, b.dz, C, {sg(M, mat(b.da, M), mat_t(b.ffg, M)), sg(M, mat(b.dbb, M), mat_t(b.ffu, M))})});
    // transition norm
    if (af3) {
        r.eg({ej(EW_COPY, N, C, b.dx1, C, b.dx2, C), ej(EW_MUL, N, C, b.gt, C, b.dz, C, b.sig[2], C),
              ej(EW_DGATE, N, C, b.dzs[2], C, b.dz, C, b.xh1, C, b.sig[2], C)});
        r.norm_bwd(0, N, C, b.xh1, b.r1, b.gt, b.dx1, 1);
    } else {
        r.eg({ej(EW_COPY, N, C, b.dx1, C, b.dx2, C),
              ej(EW_MUL1, N, C, b.gt, C, b.dz, C, b.mods + 4 * C, C6),
              ej(EW_MUL, N, C, b.dmods + 4 * C, C6, b.dz, C, b.xh1, C),
              ej(EW_COPY, N, C, b.dmods + 3 * C, C6, b.dz, C)});
        r.norm_bwd(1, N, C, b.xh1, b.r1, b.gt, b.dx1, 1);
    }
    // x1 = x0 + gA * u
    r.eg({ej(EW_MUL, N, C, b.du, C, b.dx1, C, gA, ldg),
          af3 ? ej(EW_DGATE, N, C, b.dzg[0], C, b.dx1, C, b.uu, C, b.gr[0], C)
              : ej(EW_MUL, N, C, b.dmods + 2 * C, C6, b.dx1, C, b.uu, C)});
    // output projection and value gate
    r.fork();
    r.leaf_mm(HD, C, N, mat_t(b.og, HD), mat(b.du, C), gpar ? gpar->w_attention_out : nullptr, C);
    r.mm(N, HD, C, mat(b.du, C), mat_t(b.wao, C), b.dog, HD);
    r.eg({ej(EW_MUL, N, HD, b.dO, HD, b.dog, HD, b.g, HD),
          ej(EW_DGATE, N, HD, b.dGp, HD, b.dog, HD, b.o, HD, b.g, HD)});
    prof_end(sp, s);
    // slot attention
    // with four heads the pair parameters' sums over the partial records are
    // leaves on the side stream (the records' [V] and [V][4] blocks are the
    // gradients' layouts); otherwise slot_bwd sums them itself
    const bool pw_leaf = af3 && gpar && H == 4;
    if (r.err == hipSuccess)
        r.ok(slot_bwd(sa, af3 ? STYLE_AF3 : STYLE_ESM,
                      (gpar && !pw_leaf) ? gpar->pair_scale : nullptr,
                      (gpar && !pw_leaf) ? gpar->w_pair : nullptr, s));
    if (pw_leaf && r.err == hipSuccess) {
        const int rec = slot_bwd_records(sa);
        r.fork();
        r.leaf_cs(rec, V, b.pwp, kSlotPairRecord, nullptr, 0, gpar->pair_scale);
        r.leaf_cs(rec, V * 4, b.pwp + 16, kSlotPairRecord, nullptr, 0, gpar->w_pair);
    }
    sp = prof_begin(KN_BWD_CHAIN, s);
    if (!af3 && r.err == hipSuccess)
        r.ok(head_rope_bwd(N, H, D, eps, b.qraw, b.kraw, cs_f, sn_f, b.dq, b.dk, dcos, dsin, s));
    // projections
    if (gpar) {
        r.fork();
        r.leaf_mm(C, HD, N, mat_t(b.qin, C), mat(b.dq, HD), gpar->w_q, HD);
        if (af3)
            r.leaf_cs(N, HD, b.dq, HD, nullptr, 0, gpar->b_q);
        r.leaf_mm(C, HD, N, mat_t(b.qin, C), mat(b.dGp, HD), gpar->w_value_gate, HD);
        r.leaf_mm(C, HD, N, mat_t(b.kvin, C), mat(b.dk, HD), gpar->w_k, HD);
        r.leaf_mm(C, HD, N, mat_t(b.kvin, C), mat(b.dv, HD), gpar->w_v, HD);
    }
    const GemmSeg sq = sg(HD, mat(b.dq, HD), mat_t(b.wq, HD)), sgp = sg(HD, mat(b.dGp, HD), mat_t(b.wvg, HD));
    const GemmSeg sk = sg(HD, mat(b.dk, HD), mat_t(b.wk, HD)), sv = sg(HD, mat(b.dv, HD), mat_t(b.wv, HD));
    // modulated norms
    if (af3) {
        r.mmg({gj(N, C, b.dqin, C, {sq, sgp}), gj(N, C, b.dkvin, C, {sk, sv})});
        EwJob g2 = ej(EW_FMA2, N, C, b.gt, C, b.dqin, C, b.sig[0], C, b.dkvin, C);
        g2.d = view(b.sig[1], C);
        r.eg({ej(EW_COPY, N, C, b.dx0, C, b.dx1, C), g2,
              ej(EW_DGATE, N, C, b.dzs[0], C, b.dqin, C, b.xh0, C, b.sig[0], C),
              ej(EW_DGATE, N, C, b.dzs[1], C, b.dkvin, C, b.xh0, C, b.sig[1], C)});
        r.norm_bwd(0, N, C, b.xh0, b.r0, b.gt, b.dx0, 1);
    } else {
        // q_in and kv_in are one tensor: its gradient sums all four products
        r.mmg({gj(N, C, b.dqin, C, {sq, sgp, sk, sv})});
        r.eg({ej(EW_COPY, N, C, b.dx0, C, b.dx1, C),
              ej(EW_MUL1, N, C, b.gt, C, b.dqin, C, b.mods + C, C6),
              ej(EW_MUL, N, C, b.dmods + C, C6, b.dqin, C, b.xh0, C),
              ej(EW_COPY, N, C, b.dmods, C6, b.dqin, C)});
        r.norm_bwd(1, N, C, b.xh0, b.r0, b.gt, b.dx0, 1);
    }
    // conditioning
    if (af3) {
        const float *dmu[3] = {b.dqin, b.dkvin, b.dz};
        if (gpar) {
            r.fork();
            for (int j = 0; j < 3; ++j) {
                r.leaf_mm(S, C, N, mat_t(b.cj[j], S), mat(b.dzs[j], C),
                          gpar->w_scale ? gpar->w_scale + (size_t)j * S * C : nullptr, C);
                r.leaf_mm(S, C, N, mat_t(b.cj[j], S), mat(dmu[j], C),
                          gpar->w_shift ? gpar->w_shift + (size_t)j * S * C : nullptr, C);
                r.leaf_cs(N, C, b.dzs[j], C, nullptr, 0,
                          gpar->b_scale ? gpar->b_scale + j * C : nullptr);
            }
            for (int j = 0; j < 2; ++j) {
                r.leaf_mm(S, C, N, mat_t(b.c, S), mat(b.dzg[j], C),
                          gpar->w_residual_gate ? gpar->w_residual_gate + (size_t)j * S * C : nullptr, C);
                r.leaf_cs(N, C, b.dzg[j], C, nullptr, 0,
                          gpar->b_residual_gate ? gpar->b_residual_gate + j * C : nullptr);
            }
        }
        // dc: the residual gates' part here, the conditioning norm's added below
        GemmJob js[kGroupJobs];
        int nj = 0;
        for (int j = 0; j < 3; ++j)
            js[nj++] = gj(N, S, b.dcj[j], S,
                          {sg(C, mat(b.dzs[j], C), mat_t(b.ws + (size_t)j * S * C, C)),
                           sg(C, mat(dmu[j], C), mat_t(b.wsh + (size_t)j * S * C, C))});
        js[nj++] = gj(N, S, b.dc, S,
                      {sg(C, mat(b.dzg[0], C), mat_t(b.wrg, C)),
                       sg(C, mat(b.dzg[1], C), mat_t(b.wrg + (size_t)S * C, C))});
        r.mmg(js, nj);
        EwJob m3 = ej(EW_MUL_VEC3, N, S, b.dch, S, b.dcj[0], S, b.dcj[1], S, b.dcj[2], S, b.cs);
        m3.vec2 = b.cs + S;
        m3.vec3 = b.cs + 2 * S;
        r.eg({m3});
        if (gpar && gpar->cond_scale) {
            r.fork();
            for (int j = 0; j < 3; ++j)
                r.leaf_cs(N, S, b.dcj[j], S, b.ch, S, gpar->cond_scale + j * S);
        }
        r.norm_bwd(0, N, S, b.ch, b.rc, b.dch, b.dc, 1);
    } else {
        if (gpar && gpar->w_mod) {
            r.fork();
            r.leaf_mm(S, C6, N, mat_t(b.sc, S), mat(b.dmods, C6), gpar->w_mod, C6);
        }
        r.mm(N, S, C6, mat(b.dmods, C6), mat_t(b.wmod, C6), b.ds, S);
        r.e(EW_DSILU, N, S, b.dc, S, b.ds, S, b.c, S);
    }
    {
        EwJob mk[2];
        int nm2 = 0;
        if (gin && gin->condition)
            mk[nm2++] = ej(EW_MASK, N, S, gin->condition, S, b.dc, S, nullptr, 0, nullptr, 0, nullptr,
                           b.usable);
        if (gin && gin->atom)
            mk[nm2++] = ej(EW_MASK, N, C, gin->atom, C, b.dx0, C, nullptr, 0, nullptr, 0, nullptr,
                           b.usable);
        r.eg(mk, nm2);
    }
    if (dec && ((gin && gin->token) || (gpar && gpar->w_token))) {
        if (r.err == hipSuccess)
            r.ok(token_keys(B, A, T, b.usable, in->atom_to_token, b.tkey, s));
        if (r.err == hipSuccess)
            r.ok(reverse_index(b.tkey, N, BT, b.tcnt, b.toff, b.tlist, s));
        if (r.err == hipSuccess)
            r.ok(segment_sum(BT, C, b.toff, b.tlist, b.dx0, b.dtp, s));
        if (gpar && gpar->w_token) {
            r.fork();
            r.leaf_mm(U, C, BT, mat_t(b.tok, U), mat(b.dtp, C), gpar->w_token, C);
        }
        if (gin && gin->token)
            r.mm(BT, U, C, mat(b.dtp, C), mat_t(b.wtok, C), gin->token, U);
    }
    r.join();
    prof_end(sp, s);
    return r.err == hipSuccess ? ATOM_ATTN_OK : ATOM_ATTN_ELAUNCH;
}

int check_backward(const atom_attn_dims *d, int style, int stage, int dtype) {
    if (!d || d->B < 1 || d->A < 1 || d->T < 1 || d->K < 1 || d->C < 1 || d->S < 1 ||
        d->H < 1 || d->D < 1 || d->V < 1 || d->M < 1 || d->U < 1)
        return ATOM_ATTN_EINVAL;
    if ((style != ATOM_ATTN_AF3 && style != ATOM_ATTN_ESMFOLD2) ||
        (stage != ATOM_ATTN_ENCODER && stage != ATOM_ATTN_DECODER) ||
        (dtype != ATOM_ATTN_F32 && dtype != ATOM_ATTN_BF16))
        return ATOM_ATTN_EINVAL;
    if (style == ATOM_ATTN_ESMFOLD2 && d->D % 2 != 0)
        return ATOM_ATTN_EODD_HEAD;
    return bwd_shape_ok(d, style);
}

size_t backward_bytes(const atom_attn_dims *d, int style, int stage) {
    Arena ar{nullptr};
    Bufs b;
    carve(ar, d, style, stage, b);
    return ar.off + 256;
}

} // namespace

extern "C" {

int atom_attn_backward_workspace_bytes(const atom_attn_dims *dims, int style, int stage,
                                       int dtype, size_t *bytes) {
    const int rc = check_backward(dims, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    if (!bytes)
        return ATOM_ATTN_EINVAL;
    *bytes = backward_bytes(dims, style, stage);
    return ATOM_ATTN_OK;
}

int atom_attn_backward(const atom_attn_dims *dims, int style, int stage, int dtype,
                       const atom_attn_inputs *in, const atom_attn_params *par, double eps,
                       int64_t radius, const atom_attn_grad_outputs *grad_out,
                       atom_attn_input_grads *grad_in, atom_attn_param_grads *grad_par,
                       void *workspace, size_t workspace_bytes, void *stream) {
    int rc = check_backward(dims, style, stage, dtype);
    if (rc != ATOM_ATTN_OK)
        return rc;
    if (!in || !par || !grad_out || !eps_ok(eps) || radius < -1)
        return ATOM_ATTN_EINVAL;
    const bool af3 = style == ATOM_ATTN_AF3, dec = stage == ATOM_ATTN_DECODER;
    if (!in->atom || !in->condition || !in->valid || !in->token_valid || !in->window_mask ||
        !in->atom_to_token || !in->key_index)
        return ATOM_ATTN_EINVAL;
    if (af3 && (!in->pair || !par->cond_scale || !par->w_scale || !par->b_scale ||
                !par->w_shift || !par->w_residual_gate || !par->b_residual_gate || !par->b_q ||
                !par->pair_scale || !par->w_pair))
        return ATOM_ATTN_EINVAL;
    if (!af3 && (!in->rope_cos || !in->rope_sin || !par->w_mod))
        return ATOM_ATTN_EINVAL;
    if (!par->w_q || !par->w_k || !par->w_v || !par->w_value_gate || !par->w_attention_out ||
        !par->w_ff_gate || !par->w_ff_up || !par->w_ff_out)
        return ATOM_ATTN_EINVAL;
    if (dec && (!in->token || !par->w_token || !par->readout_scale || !par->w_readout ||
                (!af3 && !par->readout_bias)))
        return ATOM_ATTN_EINVAL;
    if (!dec && !par->w_pool)
        return ATOM_ATTN_EINVAL;
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 ||
        workspace_bytes < backward_bytes(dims, style, stage))
        return ATOM_ATTN_EWORKSPACE;
    return run_backward(dims, style, stage, dtype, in, par, (float)eps, radius, grad_out, grad_in,
                        grad_par, workspace, (hipStream_t)stream);
}

int atom_attn_slot_backward_workspace_bytes(const atom_attn_dims *dims, int style,
                                            size_t *bytes) {
    if (!dims || !bytes || dims->B < 1 || dims->A < 1 || dims->K < 1 || dims->H < 1 ||
        dims->D < 1 || dims->V < 1 || (style != ATOM_ATTN_AF3 && style != ATOM_ATTN_ESMFOLD2))
        return ATOM_ATTN_EINVAL;
    const int rc = bwd_shape_ok(dims, style);
    if (rc != ATOM_ATTN_OK)
        return rc;
    const size_t N = dims->B * dims->A, E = N * dims->K, HD = dims->H * dims->D;
    Arena ar{nullptr};
    ar.get<float>(E * dims->H);                   // weights
    ar.get<float>(N * HD);                        // o
    ar.get<float>(E * dims->H);                   // logit gradients
    ar.get<int32_t>(E);                           // slot -> key
    ar.get<int32_t>(reverse_index_count_ints(N)); // reverse index
    ar.get<int32_t>(N + 1);
    ar.get<int32_t>(E);
    ar.get<int32_t>(E);                           // list position of each entry
    ar.get<float>(E * dims->H);                   // key-major weights
    ar.get<int32_t>(slot_bwd_queue_ints(dims->B, dims->A)); // wide blocks
    ar.get<float>(slot_bwd_partial_floats(dims->B, dims->A, (int)dims->V, (int)dims->H));
    ar.get<float>(dims->V);                       // pair parameters in fp32
    ar.get<float>(dims->V * dims->H);
    ar.get<float>(slot_bwd_partial_floats(dims->B, dims->A, (int)dims->V, (int)dims->H)); // sums
    *bytes = ar.off + 256;
    return ATOM_ATTN_OK;
}

int atom_attn_slot_attention_backward(const atom_attn_dims *dims, int style, int dtype,
                                      double eps, int64_t radius, const uint8_t *usable,
                                      const float *q, const float *k, const float *v,
                                      const int64_t *key_index, const uint8_t *window_mask,
                                      const void *pair, const void *pair_scale,
                                      const void *w_pair, const float *d_attention,
                                      const float *d_o, float *attention, float *o, float *dq,
                                      float *dk, float *dv, float *d_pair, float *d_pair_scale,
                                      float *d_w_pair, void *workspace, size_t workspace_bytes,
                                      void *stream) {
    size_t need = 0;
    int rc = atom_attn_slot_backward_workspace_bytes(dims, style, &need);
    if (rc != ATOM_ATTN_OK)
        return rc;
    const bool af3 = style == ATOM_ATTN_AF3;
    if ((dtype != ATOM_ATTN_F32 && dtype != ATOM_ATTN_BF16) || !eps_ok(eps) || radius < -1 ||
        !usable || !q || !k || !v || !key_index || !window_mask || !d_o || !dq || !dk || !dv)
        return ATOM_ATTN_EINVAL;
    if (af3 && (!pair || !pair_scale || !w_pair))
        return ATOM_ATTN_EINVAL;
    const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v;
    if (al & 15u)
        return ATOM_ATTN_EINVAL;
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < need)
        return ATOM_ATTN_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const size_t N = dims->B * dims->A, E = N * dims->K, HD = dims->H * dims->D;
    Arena ar{(char *)workspace};
    float *P = ar.get<float>(E * dims->H);
    float *ob = ar.get<float>(N * HD);
    float *dS = ar.get<float>(E * dims->H);
    int32_t *kid = ar.get<int32_t>(E);
    int32_t *cnt = ar.get<int32_t>(reverse_index_count_ints(N));
    int32_t *off = ar.get<int32_t>(N + 1);
    int32_t *list = ar.get<int32_t>(E);
    int32_t *inv = ar.get<int32_t>(E);
    float *Pk = ar.get<float>(E * dims->H);
    int32_t *wq = ar.get<int32_t>(slot_bwd_queue_ints(dims->B, dims->A));
    float *pwp = ar.get<float>(slot_bwd_partial_floats(dims->B, dims->A, (int)dims->V, (int)dims->H));
    float *psf = ar.get<float>(dims->V);              // pair parameters in fp32
    float *wpf = ar.get<float>(dims->V * dims->H);
    const size_t pcap = slot_bwd_partial_floats(dims->B, dims->A, (int)dims->V, (int)dims->H);
    float *cpart = ar.get<float>(pcap);
    const Scratch sc{cpart, pcap};
    hipError_t e = hipSuccess;
    SlotBwdArgs sa{};
    sa.B = (int)dims->B; sa.A = (int)dims->A; sa.K = (int)dims->K; sa.H = (int)dims->H;
    sa.D = (int)dims->D; sa.V = (int)dims->V; sa.eps = (float)eps; sa.radius = radius;
    sa.pair_dtype = dtype; sa.usable = usable; sa.window_mask = window_mask;
    sa.key_index = key_index; sa.q = q; sa.k = k; sa.v = v; sa.pair = af3 ? pair : nullptr;
    sa.ps = psf; sa.wp = wpf; sa.P = attention ? attention : P; sa.o = o ? o : ob;
    sa.kid = kid; sa.d_att = d_attention; sa.d_o = d_o; sa.dS = dS; sa.dq = dq; sa.dk = dk;
    sa.dv = dv; sa.d_pair = af3 ? d_pair : nullptr; sa.pw_partial = pwp; sa.count = cnt;
    sa.offset = off; sa.list = list; sa.sc = sc; sa.inv = inv; sa.Pk = Pk; sa.wide = wq;
    if (af3 && e == hipSuccess) {
        e = to_f32(pair_scale, dtype, 1, (int)dims->V, dims->V, psf, nullptr, s);
        if (e == hipSuccess)
            e = to_f32(w_pair, dtype, 1, (int)(dims->V * dims->H), dims->V * dims->H, wpf,
                       nullptr, s);
    }
    if (e == hipSuccess) {
        ProfSpan sp = prof_begin(KN_BWD_SLOT_FWD, s);
        e = slot_fwd(sa, af3 ? STYLE_AF3 : STYLE_ESM, s);
        prof_end(sp, s);
    }
    if (e == hipSuccess)
        e = slot_bwd(sa, af3 ? STYLE_AF3 : STYLE_ESM, af3 ? d_pair_scale : nullptr,
                     af3 ? d_w_pair : nullptr, s);
    return e == hipSuccess ? ATOM_ATTN_OK : ATOM_ATTN_ELAUNCH;
}

} // extern "C"
