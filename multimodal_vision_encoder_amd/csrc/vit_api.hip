// Host side of the C ABI: validation, batch planning, weight preparation, workspace and the
// launch sequence of one encoder pass.  Every argument of a call is checked before anything
// is enqueued ([L] DS4V: failed multi-image encoding publishes no partial embeddings).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "loaders.h"
#include "vit.h"
#include "vit_ops.h"

constexpr size_t kNoAllocScratchBytes = (size_t)256 * 256 * 128 * sizeof(float);   // 32 MiB
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxSide = 4096;       // largest patch-grid side (rows of the RoPE tables)
constexpr int kMaxImages = 4096;     // images per call
constexpr int kVtAlign = 64;         // per-image column alignment of the transposed-V buffer

thread_local std::string g_err;

// Fixed device scratch of vit_op_linear_noalloc: the fp32 split-K partial tiles of one GEMM
// launch (at most one 256 x 128 tile per compute unit of a 256-CU GPU).  Every GPU the library
// runs on holds its own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: its device address is resolved per device with
// hipGetSymbolAddress (scratch_on_device) and only that address is passed to kernels.
constexpr int kMaxDevices = 64;
float *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of `scratch` on device `dev` (resolved once per device, with that device
// current); NULL with *err set if it cannot be resolved.
float *scratch_on_device(int dev, hipError_t *err)
{
    *err = hipSuccess;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch_ptr[dev] = (float *)p;
    }
    return g_scratch_ptr[dev];
}

// Per-layer weights.  With the SwiGLU MLP, w1/b1 are the gate and up rows interleaved in
// groups of 8 (the ACT_SWIGLU layout, 2F rows) and w2/b2 the down projection; with RMSNorm the
// norms have no beta (ln1b, ln2b NULL).
struct Layer {
    const bf16_t *ln1g, *ln1b, *wqkv, *bqkv, *wo, *bo, *ln2g, *ln2b, *w1, *b1, *w2, *b2;
};

struct Plan {
    std::vector<ImgDesc> imgs;
    std::vector<RowTile> attn, rope;
    int64_t N = 0, M = 0, vt_cols = 0;
    int64_t npx = 0;   // pixel bytes of the batch
};

}  // namespace

struct vit_ctx {
    vit_config cfg{};
    int device = 0;
    int D = 0, H = 0, hd = 0, F = 0, Dl = 0, L = 0, ps = 0, Kp = 0;
    float s3[3] = {0, 0, 0}, t3[3] = {0, 0, 0};

    bf16_t *d_blob = nullptr, *d_wpe = nullptr, *d_wproj = nullptr;
    bf16_t *d_gu = nullptr;            // SwiGLU: interleaved gate/up weights and biases of all layers
    const bf16_t *wproj2 = nullptr, *proj2_b = nullptr;   // second aligner projection
    int Da = 0;                        // rows of the first aligner projection
    bf16_t *a1 = nullptr;              // aligner inner activations, bf16 [cap_tokens][Da]
    int64_t cap_tokens = 0;
    bf16_t *d_zero = nullptr;   // 256 zero bytes: the padding source of the merge gather
    uint8_t *d_tinypx = nullptr; // 64 bytes: padded copy of a batch of fewer than 12 pixel bytes
    uint16_t *d_sentinels = nullptr;   // learned START, NEWLINE, END rows, bf16 [3][Dl]
    float *d_pre_ws = nullptr;         // preprocessing scratch (horizontal resize pass)
    size_t pre_ws_bytes = 0;
    const bf16_t *pe_b = nullptr, *lnf_g = nullptr, *lnf_b = nullptr, *proj_b = nullptr;
    std::vector<Layer> layers;
    float *d_cos = nullptr, *d_sin = nullptr;

    // workspace
    float *d_gemm_ws = nullptr;   // split-K partial tiles of the GEMMs
    size_t gemm_ws_bytes = 0;
    char *d_attn_ws = nullptr;    // key-slice partials of the attention
    size_t attn_ws_bytes = 0;
    int attn_split_fixed = 0;     // 0: chosen per batch; 1..4: fixed key slices
    int span_layout = VIT_SPAN_V41;   // span geometry of vit_assemble
    int64_t cap_patches = 0, cap_vt_cols = 0, reserve_cap = 0;
    bf16_t *x = nullptr, *ln = nullptr, *qkv = nullptr, *vt = nullptr, *o = nullptr, *h1 = nullptr;

    // per-call metadata: pinned staging -> device
    char *h_stage = nullptr, *d_meta = nullptr;
    size_t meta_cap = 0;
    hipEvent_t stage_ev = nullptr;
    bool stage_pending = false;

    // optional per-step timing (event pairs recorded around launches)
    bool timing = false;
    std::vector<hipEvent_t> ev_pool;
    size_t ev_next = 0;
    std::vector<std::pair<int, size_t>> ev_marks;   // (step kind, index of the start event)

    std::string err;
};

namespace {

vit_status fail(vit_ctx *ctx, vit_status st, const std::string &msg)
{
    (ctx ? ctx->err : g_err) = msg;
    return st;
}

#define HIP_TRY(ctx, expr)                                                                    \
    do {                                                                                      \
        hipError_t e_ = (expr);                                                               \
        if (e_ != hipSuccess)                                                                 \
            return fail(ctx, VIT_E_DEVICE, std::string(#expr) + ": " + hipGetErrorString(e_)); \
    } while (0)

bool supported_hidden(int D)
{
    return D == 64 || D == 128 || D == 256 || D == 512 || D == 1024 || D == 1536 || D == 2048;
}

std::string check_config(const vit_config &c)
{
    if (c.layers < 0) return "layers < 0";
    if (!supported_hidden(c.hidden)) return "hidden must be one of 64,128,256,512,1024,1536,2048";
    if (c.heads < 1 || c.hidden % c.heads) return "heads must divide hidden";
    const int hd = c.hidden / c.heads;
    if (hd != 16 && hd != 32 && hd != 64 && hd != 128) return "head_dim must be 16, 32, 64 or 128";
    if (c.mlp < 64 || c.mlp % 64) return "mlp must be a positive multiple of 64";
    if (c.patch < 1 || c.patch > 64) return "patch must be in [1, 64]";
    if (c.merge != 3) return "merge must be 3";
    if (c.out_hidden < 1) return "out_hidden must be >= 1";
    if (c.max_tokens_per_image < 1) return "max_tokens_per_image must be >= 1";
    if (!(c.ln_eps > 0.f) || !(c.rope_base > 0.f)) return "ln_eps and rope_base must be > 0";
    if (c.norm_kind != 0 && c.norm_kind != 1) return "norm_kind must be 0 or 1";
    if (c.mlp_kind != 0 && c.mlp_kind != 1) return "mlp_kind must be 0 or 1";
    if (c.gelu_kind != 0 && c.gelu_kind != 1) return "gelu_kind must be 0 or 1";
    if (c.aligner_hidden < 0 || c.aligner_hidden % 64) return "aligner_hidden must be 0 or a positive multiple of 64";
    for (int i = 0; i < 3; ++i)
        if (!(c.pix_std[i] != 0.f) || !std::isfinite(c.pix_std[i]) || !std::isfinite(c.pix_mean[i]))
            return "pixel std must be non-zero and finite";
    return "";
}

size_t blob_elems_of(const vit_config &c)
{
    const size_t D = c.hidden, F = c.mlp, P = 3 * (size_t)c.patch * c.patch, Dl = c.out_hidden;
    const size_t nrm = c.norm_kind == 1 ? D : 2 * D;                 // gamma (+ beta)
    const size_t mlp = c.mlp_kind == 1 ? 3 * F * D + 2 * F + D : 2 * F * D + F + D;
    const size_t Da = c.aligner_hidden;
    size_t n = D * P + D;
    n += (size_t)c.layers * (2 * nrm + 3 * D * D + 3 * D + D * D + D + mlp);
    n += nrm + (Da ? Da * 9 * D + Da + Dl * Da + Dl : Dl * 9 * D + Dl);
    return n;
}

int gelu_act(const vit_config &c) { return c.gelu_kind == 1 ? ACT_GELU_ERF : ACT_GELU_TANH; }

int64_t tokens_of(int gh, int gw) { return (int64_t)((gh + 2) / 3) * ((gw + 2) / 3); }

constexpr int kSpanAlign = 4;    // V4 Flash spans: positions in groups of 4 ([G] pos % 4)

// Positions of one image's span: V4.1, START + mh (mw IMAGE + NEWLINE) + END; V4 Flash
// (reading of [G]: row-pair interleave, pos % 4 alignment, compress_pad), START + per pair of
// merged rows its 2 mw (or mw for a last lone row) IMAGE and one NEWLINE + END, then PAD up to
// a multiple of 4.
int64_t span_length(int layout, int64_t mh, int64_t mw)
{
    if (layout != VIT_SPAN_V4) return 2 + mh * (mw + 1);
    const int64_t core = 2 + (mh + 1) / 2 + mh * mw;
    return (core + kSpanAlign - 1) / kSpanAlign * kSpanAlign;
}

// Type of position k of an image's span and, for IMAGE, the merged token (r * mw + c) it takes.
int span_entry(int layout, int64_t mh, int64_t mw, int64_t k, int64_t *tok)
{
    *tok = -1;
    if (k == 0) return VIT_TOK_START;
    if (layout != VIT_SPAN_V4) {
        if (k == 1 + mh * (mw + 1)) return VIT_TOK_END;
        const int64_t q = k - 1, r = q / (mw + 1), c = q - r * (mw + 1);
        if (c == mw) return VIT_TOK_NEWLINE;
        *tok = r * mw + c;
        return VIT_TOK_IMAGE;
    }
    const int64_t core = 2 + (mh + 1) / 2 + mh * mw;
    if (k == core - 1) return VIT_TOK_END;
    if (k >= core) return VIT_TOK_PAD;
    const int64_t q = k - 1, pairs = mh / 2, pair_len = 2 * mw + 1;
    if (q < pairs * pair_len) {
        const int64_t p = q / pair_len, j = q - p * pair_len;
        if (j == 2 * mw) return VIT_TOK_NEWLINE;
        *tok = (2 * p + (j & 1)) * mw + j / 2;
        return VIT_TOK_IMAGE;
    }
    const int64_t j = q - pairs * pair_len;   // the last, lone merged row
    if (j == mw) return VIT_TOK_NEWLINE;
    *tok = (mh - 1) * mw + j;
    return VIT_TOK_IMAGE;
}

vit_status make_plan(vit_ctx *ctx, const vit_grid *grids, int n, Plan &p)
{
    if (n < 0 || n > kMaxImages) return fail(ctx, VIT_E_ARG, "n_images out of range");
    if (n > 0 && !grids) return fail(ctx, VIT_E_ARG, "h_grids is NULL");
    p = Plan();
    int64_t pix = 0;
    for (int i = 0; i < n; ++i) {
        const int gh = grids[i].gh, gw = grids[i].gw;
        if (gh < 1 || gw < 1 || gh > kMaxSide || gw > kMaxSide)
            return fail(ctx, VIT_E_ARG, "image " + std::to_string(i) + ": grid " +
                                            std::to_string(gh) + "x" + std::to_string(gw) +
                                            " out of range [1, " + std::to_string(kMaxSide) + "]");
        const int64_t tok = tokens_of(gh, gw);
        if (tok > ctx->cfg.max_tokens_per_image)
            return fail(ctx, VIT_E_BUDGET, "image " + std::to_string(i) + ": " + std::to_string(tok) +
                                               " merged tokens exceed the budget of " +
                                               std::to_string(ctx->cfg.max_tokens_per_image));
        ImgDesc d{};
        d.gh = gh;
        d.gw = gw;
        d.n = gh * gw;
        d.patch_off = (int32_t)p.N;
        d.tok_off = (int32_t)p.M;
        d.mh = (gh + 2) / 3;
        d.mw = (gw + 2) / 3;
        d.vt_off = (int32_t)p.vt_cols;
        d.pix_off = pix;
        p.imgs.push_back(d);
        p.N += d.n;
        p.M += tok;
        p.vt_cols += ceil_div(d.n, kVtAlign) * kVtAlign;
        pix += (int64_t)ctx->ps * gh * ctx->ps * gw * 3;
        if (p.vt_cols > INT32_MAX / 2) return fail(ctx, VIT_E_ARG, "batch too large");
    }
    p.npx = pix;
    // attention query tiles, largest images first (longest-processing-time order)
    std::vector<int> order(n);
    for (int i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return p.imgs[a].n > p.imgs[b].n; });
    const int qt = attention_q_tile();
    for (int i : order)
        for (int r = 0; r < p.imgs[i].n; r += qt) p.attn.push_back(RowTile{i, r});
    for (int i = 0; i < n; ++i)
        for (int r = 0; r < p.imgs[i].n; r += kRopeTile) p.rope.push_back(RowTile{i, r});
    return VIT_OK;
}

void free_workspace(vit_ctx *c)
{
    bf16_t **bufs[] = {&c->x, &c->ln, &c->qkv, &c->vt, &c->o, &c->h1};
    for (auto b : bufs) {
        if (*b) (void)hipFree(*b);
        *b = nullptr;
    }
    c->cap_patches = c->cap_vt_cols = 0;
}

// Split-K scratch of the GEMMs, allocated once at its largest size.  Without it (allocation
// failed) the GEMMs run unsplit, which gives the same results.
GemmWorkspace gemm_ws(vit_ctx *c)
{
    if (!c->d_gemm_ws) {
        const size_t bytes = gemm_workspace_max_bytes();
        if (hipMalloc((void **)&c->d_gemm_ws, bytes) == hipSuccess) {
            c->gemm_ws_bytes = bytes;
        } else {
            (void)hipGetLastError();
            c->d_gemm_ws = nullptr;
        }
    }
    return GemmWorkspace{c->d_gemm_ws, c->d_gemm_ws ? c->gemm_ws_bytes : 0};
}

// Attention work split for this batch and its scratch (grown on demand; without it the
// attention runs unsplit, which gives results within the same bounds).
AttnSplit attn_split(vit_ctx *c, const Plan &p)
{
    AttnSplit sp = attention_plan(p.imgs.data(), (int)p.imgs.size(), (int)p.attn.size(), c->D, c->H,
                                  c->attn_split_fixed);
    const size_t need = attention_plan_bytes(sp, c->D, c->H);
    auto unsplit = [&]() {
        sp.full = sp.per_xcd;
        sp.slices = 1;
        return sp;
    };
    if (need == 0) return unsplit();
    if (need > c->attn_ws_bytes) {
        if (hipDeviceSynchronize() != hipSuccess) {
            (void)hipGetLastError();
            return unsplit();
        }
        if (c->d_attn_ws) (void)hipFree(c->d_attn_ws);
        c->d_attn_ws = nullptr;
        c->attn_ws_bytes = 0;
        if (hipMalloc((void **)&c->d_attn_ws, need) != hipSuccess) {
            (void)hipGetLastError();
            c->d_attn_ws = nullptr;
            return unsplit();
        }
        c->attn_ws_bytes = need;
    }
    const size_t rows = (size_t)8 * (sp.per_xcd - sp.full) * sp.slices * attention_q_tile();
    sp.part_o = (uint16_t *)c->d_attn_ws;
    sp.part_ml = (float *)(c->d_attn_ws + rows * (c->D / c->H) * sizeof(uint16_t));
    return sp;
}

vit_status ensure_workspace(vit_ctx *c, int64_t N, int64_t vt_cols)
{
    (void)gemm_ws(c);
    if (N <= c->cap_patches && vt_cols <= c->cap_vt_cols) return VIT_OK;
    if (c->reserve_cap > 0 && N > c->reserve_cap)
        return fail(c, VIT_E_NOMEM, "batch of " + std::to_string(N) +
                                        " patches exceeds the reserved workspace of " +
                                        std::to_string(c->reserve_cap));
    HIP_TRY(c, hipDeviceSynchronize());
    free_workspace(c);
    const int64_t Np = std::max<int64_t>(N, 64);
    const int64_t Vc = std::max<int64_t>(vt_cols, kVtAlign);
    const size_t D = c->D;
    struct { bf16_t **p; size_t n; } req[] = {
        {&c->x, Np * D}, {&c->ln, Np * D}, {&c->qkv, Np * 3 * D}, {&c->o, Np * D},
        {&c->h1, Np * (size_t)c->F}, {&c->vt, (size_t)c->H * c->hd * Vc}};
    for (auto &r : req) {
        if (hipMalloc((void **)r.p, r.n * sizeof(bf16_t)) != hipSuccess) {
            (void)hipGetLastError();
            free_workspace(c);
            return fail(c, VIT_E_NOMEM, "workspace allocation failed");
        }
    }
    HIP_TRY(c, hipMemset(c->vt, 0, (size_t)c->H * c->hd * Vc * sizeof(uint16_t)));
    c->cap_patches = Np;
    c->cap_vt_cols = Vc;
    return VIT_OK;
}

// Copy `bytes` of host metadata to the context's device metadata buffer on `s`.
vit_status upload_meta(vit_ctx *c, const std::vector<std::pair<const void *, size_t>> &parts,
                       hipStream_t s, std::vector<size_t> &offsets)
{
    size_t total = 0;
    offsets.clear();
    for (auto &p : parts) {
        offsets.push_back(total);
        total += (p.second + 255) & ~(size_t)255;
    }
    if (total == 0) return VIT_OK;
    if (c->stage_pending) {
        HIP_TRY(c, hipEventSynchronize(c->stage_ev));
        c->stage_pending = false;
    }
    if (total > c->meta_cap) {
        HIP_TRY(c, hipDeviceSynchronize());
        if (c->h_stage) (void)hipHostFree(c->h_stage);
        if (c->d_meta) (void)hipFree(c->d_meta);
        c->h_stage = c->d_meta = nullptr;
        c->meta_cap = 0;
        const size_t cap = std::max<size_t>(total, 1 << 16);
        if (hipHostMalloc((void **)&c->h_stage, cap, hipHostMallocDefault) != hipSuccess ||
            hipMalloc((void **)&c->d_meta, cap) != hipSuccess) {
            (void)hipGetLastError();
            return fail(c, VIT_E_NOMEM, "metadata staging allocation failed");
        }
        c->meta_cap = cap;
    }
    for (size_t i = 0; i < parts.size(); ++i)
        if (parts[i].second) std::memcpy(c->h_stage + offsets[i], parts[i].first, parts[i].second);
    HIP_TRY(c, hipMemcpyAsync(c->d_meta, c->h_stage, total, hipMemcpyHostToDevice, s));
    HIP_TRY(c, hipEventRecord(c->stage_ev, s));
    c->stage_pending = true;
    return VIT_OK;
}

struct DevPlan {
    const ImgDesc *imgs;
    const RowTile *attn, *rope;
};

vit_status stage_plan(vit_ctx *c, const Plan &p, hipStream_t s, DevPlan &dp)
{
    std::vector<size_t> off;
    vit_status st = upload_meta(c,
                                {{p.imgs.data(), p.imgs.size() * sizeof(ImgDesc)},
                                 {p.attn.data(), p.attn.size() * sizeof(RowTile)},
                                 {p.rope.data(), p.rope.size() * sizeof(RowTile)}},
                                s, off);
    if (st != VIT_OK) return st;
    dp.imgs = (const ImgDesc *)(c->d_meta + off[0]);
    dp.attn = (const RowTile *)(c->d_meta + off[1]);
    dp.rope = (const RowTile *)(c->d_meta + off[2]);
    return VIT_OK;
}

#define LAUNCH(ctx, expr)                                                                     \
    do {                                                                                      \
        hipError_t e_ = (expr);                                                               \
        if (e_ != hipSuccess)                                                                 \
            return fail(ctx, VIT_E_DEVICE, std::string("launch failed: ") + #expr + ": " +    \
                                               hipGetErrorString(e_));                        \
    } while (0)

// Record the start event of a timed launch; returns the pool index or -1 when not timing.
long timing_start(vit_ctx *c, hipStream_t s)
{
    if (!c->timing) return -1;
    if (c->ev_next + 2 > c->ev_pool.size()) {
        for (int i = 0; i < 256; ++i) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) return -1;
            c->ev_pool.push_back(e);
        }
    }
    const size_t i = c->ev_next;
    if (hipEventRecord(c->ev_pool[i], s) != hipSuccess) return -1;
    c->ev_next += 2;
    return (long)i;
}

void timing_stop(vit_ctx *c, hipStream_t s, int kind, long i)
{
    if (i < 0) return;
    if (hipEventRecord(c->ev_pool[i + 1], s) == hipSuccess) c->ev_marks.push_back({kind, (size_t)i});
}

// LAUNCH with an event pair around it when timing is enabled.
#define TLAUNCH(ctx, kind, s, expr)                                                           \
    do {                                                                                      \
        const long t_ = timing_start(ctx, s);                                                 \
        LAUNCH(ctx, expr);                                                                    \
        timing_stop(ctx, s, kind, t_);                                                        \
    } while (0)

// Inner rows of the two-projection aligner: bf16 [M][Da], grown on demand; after vit_reserve
// it holds as many rows as the reserved patches (a batch never has more merged tokens than
// patches), so reserved calls do not allocate.
vit_status ensure_tokens(vit_ctx *c, int64_t M)
{
    if (!c->wproj2 || M <= c->cap_tokens) return VIT_OK;
    if (c->reserve_cap > 0 && M > c->reserve_cap)
        return fail(c, VIT_E_NOMEM, "batch of " + std::to_string(M) + " tokens exceeds the reserved workspace");
    HIP_TRY(c, hipDeviceSynchronize());
    if (c->a1) (void)hipFree(c->a1);
    c->a1 = nullptr;
    c->cap_tokens = 0;
    const int64_t cap = std::max<int64_t>(M, 64);
    if (hipMalloc((void **)&c->a1, (size_t)cap * c->Da * sizeof(bf16_t)) != hipSuccess) {
        (void)hipGetLastError();
        c->a1 = nullptr;
        return fail(c, VIT_E_NOMEM, "aligner workspace allocation failed");
    }
    c->cap_tokens = cap;
    return VIT_OK;
}

// The aligner: 3x3 merge gather + one projection into fp32 rows, or with a second projection
// bf16(GELU(first)) into the inner buffer (grown on demand), then the second into fp32.
vit_status run_aligner(vit_ctx *c, const bf16_t *y, const ImgDesc *imgs, int ni, int64_t M, float *out,
                       const GemmWorkspace *gws, hipStream_t s)
{
    if (!c->wproj2) {
        LAUNCH(c, launch_merge_project(y, imgs, ni, M, c->D, c->d_wproj, c->proj_b, c->Dl, ACT_NONE, true, out,
                                       c->d_zero, gws, s));
        return VIT_OK;
    }
    vit_status st = ensure_tokens(c, M);
    if (st != VIT_OK) return st;
    LAUNCH(c, launch_merge_project(y, imgs, ni, M, c->D, c->d_wproj, c->proj_b, c->Da, gelu_act(c->cfg), false,
                                   c->a1, c->d_zero, gws, s));
    LAUNCH(c, launch_linear(c->a1, M, c->Da, c->wproj2, c->proj2_b, c->Dl, ACT_NONE, true, out, gws, s));
    return VIT_OK;
}

constexpr int kStopNone = -1;

// One encoder pass; with stop >= 0 it ends at that debug boundary and copies the tensor.
vit_status encode_impl(vit_ctx *c, const uint8_t *px, const vit_grid *grids, int n, float *out,
                       hipStream_t s, int stop, int arg, void *dst, size_t dst_bytes)
{
    Plan p;
    vit_status st = make_plan(c, grids, n, p);
    if (st != VIT_OK) return st;
    const int D = c->D, H = c->H, L = c->L;
    const bool rms = c->cfg.norm_kind == 1, swiglu = c->cfg.mlp_kind == 1;
    const size_t b2 = sizeof(bf16_t);
    if (stop == kStopNone) {
        if (p.N > 0 && (!px || !out)) return fail(c, VIT_E_ARG, "d_pixels or d_out_rows is NULL");
    } else {
        size_t want = 0;
        switch (stop) {
        case VIT_DUMP_PATCHES: want = (size_t)p.N * 3 * c->ps * c->ps * b2; break;
        case VIT_DUMP_EMBED: case VIT_DUMP_ATTN: case VIT_DUMP_LAYER: case VIT_DUMP_FINAL_NORM:
            want = (size_t)p.N * D * b2; break;
        case VIT_DUMP_QKV: want = (size_t)p.N * 3 * D * b2; break;
        case VIT_DUMP_MERGED: want = (size_t)p.M * 9 * D * b2; break;
        case VIT_DUMP_ROPE: want = (size_t)p.N * c->hd * sizeof(float); break;
        default: return fail(c, VIT_E_ARG, "unknown dump boundary");
        }
        if ((stop == VIT_DUMP_QKV || stop == VIT_DUMP_ATTN || stop == VIT_DUMP_LAYER) &&
            (arg < 0 || arg >= L))
            return fail(c, VIT_E_ARG, "layer index out of range");
        if (dst_bytes != want) return fail(c, VIT_E_ARG, "dst_bytes does not match the boundary size");
        if (p.N > 0 && !dst) return fail(c, VIT_E_ARG, "d_dst is NULL");
        if (p.N > 0 && stop != VIT_DUMP_ROPE && !px) return fail(c, VIT_E_ARG, "d_pixels is NULL");
        if (stop == VIT_DUMP_ROPE && ((uintptr_t)dst & 15) != 0)
            return fail(c, VIT_E_ARG, "d_dst of the RoPE dump must be 16-byte aligned");
    }
    if (p.N == 0) return VIT_OK;
    st = ensure_workspace(c, p.N, p.vt_cols);
    if (st != VIT_OK) return st;
    const GemmWorkspace gws = gemm_ws(c);
    const AttnSplit asp = attn_split(c, p);
    DevPlan dp{};
    st = stage_plan(c, p, s, dp);
    if (st != VIT_OK) return st;
    const int ni = (int)p.imgs.size();
    auto copy_out = [&](const void *src) -> vit_status {
        HIP_TRY(c, hipMemcpyAsync(dst, src, dst_bytes, hipMemcpyDeviceToDevice, s));
        return VIT_OK;
    };

    if (stop == VIT_DUMP_ROPE) {
        LAUNCH(c, launch_dump_rope(dp.imgs, ni, p.N, c->hd, c->d_cos, c->d_sin, (float *)dst, s));
        return VIT_OK;
    }
    // The fused patch loader addresses under 2^31 pixel bytes per launch: whole images in
    // groups.  It reads 12 bytes per chunk, so a group of fewer than 12 pixel bytes (plus the
    // misalignment of its start) is read from a padded 64-byte copy.
    auto pixel_groups = [&](auto &&fn) -> vit_status {
        for (int i0 = 0; i0 < ni;) {
            int i1 = i0 + 1;
            const int64_t first = p.imgs[i0].pix_off;
            auto end_of = [&](int i) { return i + 1 < ni ? p.imgs[i + 1].pix_off : p.npx; };
            while (i1 < ni && end_of(i1) - first < kPatchLaunchBytes) ++i1;
            const int64_t m0 = p.imgs[i0].patch_off, m1 = i1 < ni ? p.imgs[i1].patch_off : p.N;
            const int64_t bytes = end_of(i1 - 1) - first;
            const uint8_t *lpx = px + first;
            if (bytes + (int64_t)((uintptr_t)lpx & 3) < 12) {
                HIP_TRY(c, hipMemcpyAsync(c->d_tinypx, lpx, (size_t)bytes, hipMemcpyDeviceToDevice, s));
                lpx = c->d_tinypx;
            }
            const vit_status st2 = fn(lpx, first, bytes, m0, m1 - m0);
            if (st2 != VIT_OK) return st2;
            i0 = i1;
        }
        return VIT_OK;
    };
    if (stop == VIT_DUMP_PATCHES)
        return pixel_groups([&](const uint8_t *lpx, int64_t pf, int64_t pb, int64_t m0, int64_t rows) -> vit_status {
            LAUNCH(c, launch_dump_patches(lpx, pf, pb, dp.imgs, ni, m0, rows, c->s3, c->t3, c->ps, (bf16_t *)dst, s));
            return VIT_OK;
        });
    {
        const long t_ = timing_start(c, s);
        st = pixel_groups([&](const uint8_t *lpx, int64_t pf, int64_t pb, int64_t m0, int64_t rows) -> vit_status {
            LAUNCH(c, launch_patch_embed(lpx, pf, pb, dp.imgs, ni, m0, rows, c->s3, c->t3, c->ps, c->d_wpe, c->Kp,
                                         c->pe_b, D, c->x, &gws, s));
            return VIT_OK;
        });
        if (st != VIT_OK) return st;
        timing_stop(c, s, VIT_STEP_PATCH_EMBED, t_);
    }
    if (stop == VIT_DUMP_EMBED) return copy_out(c->x);

    // the transposed-V columns past each image's end are read as masked keys: zero them once
    if (L > 0) LAUNCH(c, launch_vt_tail_zero(c->vt, p.vt_cols, dp.imgs, ni, D, s));
    for (int l = 0; l < L; ++l) {
        const Layer &w = c->layers[l];
        TLAUNCH(c, VIT_STEP_LAYERNORM, s, launch_layernorm(c->x, nullptr, nullptr, p.N, D, w.ln1g, w.ln1b,
                                   c->cfg.ln_eps, rms, c->ln, s));
        // QKV projection with RoPE on q, k and the V^T relayout in its epilogue
        TLAUNCH(c, VIT_STEP_QKV, s, launch_qkv_rope(c->ln, p.N, D, H, w.wqkv, w.bqkv, c->qkv, c->vt, p.vt_cols,
                                                    dp.imgs, ni, c->d_cos, c->d_sin,
                                                    stop == VIT_DUMP_QKV && arg == l, s));
        if (stop == VIT_DUMP_QKV && arg == l) return copy_out(c->qkv);
        TLAUNCH(c, VIT_STEP_ATTENTION, s, launch_attention(c->qkv, c->vt, p.vt_cols, c->o, dp.attn, (int)p.attn.size(),
                                   dp.imgs, D, H, asp, s));
        if (attention_needs_merge(asp))
            TLAUNCH(c, VIT_STEP_ATTN_MERGE, s,
                    launch_attention_merge(c->o, dp.attn, (int)p.attn.size(), dp.imgs, D, H, asp, s));
        if (stop == VIT_DUMP_ATTN && arg == l) return copy_out(c->o);
        // the residual adds run in the epilogues of the out-projection and fc2 (x updated in place)
        TLAUNCH(c, VIT_STEP_OUT_PROJ, s, launch_linear_residual(c->o, p.N, D, w.wo, w.bo, D, c->x, &gws, s));
        TLAUNCH(c, VIT_STEP_LAYERNORM, s, launch_layernorm(c->x, nullptr, nullptr, p.N, D, w.ln2g, w.ln2b, c->cfg.ln_eps,
                                   rms, c->ln, s));
        // GELU MLP: fc1 + GELU; SwiGLU: gate and up projections + silu(g) u in one launch
        if (swiglu)
            TLAUNCH(c, VIT_STEP_FC1, s, launch_linear(c->ln, p.N, D, w.w1, w.b1, 2 * c->F, ACT_SWIGLU, false, c->h1, &gws, s));
        else
            TLAUNCH(c, VIT_STEP_FC1, s, launch_linear(c->ln, p.N, D, w.w1, w.b1, c->F, gelu_act(c->cfg), false, c->h1, &gws, s));
        TLAUNCH(c, VIT_STEP_FC2, s, launch_linear_residual(c->h1, p.N, c->F, w.w2, w.b2, D, c->x, &gws, s));
        if (stop == VIT_DUMP_LAYER && arg == l) return copy_out(c->x);
    }
    TLAUNCH(c, VIT_STEP_LAYERNORM, s, launch_layernorm(c->x, nullptr, nullptr, p.N, D, c->lnf_g, c->lnf_b,
                               c->cfg.ln_eps, rms, c->ln, s));
    if (stop == VIT_DUMP_FINAL_NORM) return copy_out(c->ln);
    if (stop == VIT_DUMP_MERGED) {
        LAUNCH(c, launch_dump_merged(c->ln, dp.imgs, ni, p.M, D, (bf16_t *)dst, c->d_zero, s));
        return VIT_OK;
    }
    const long t_ = timing_start(c, s);
    if ((st = run_aligner(c, c->ln, dp.imgs, ni, p.M, out, &gws, s)) != VIT_OK) return st;
    timing_stop(c, s, VIT_STEP_PROJECTOR, t_);
    return VIT_OK;
}

void destroy(vit_ctx *c)
{
    if (!c) return;
    (void)hipDeviceSynchronize();
    free_workspace(c);
    void *bufs[] = {c->d_blob, c->d_wpe, c->d_wproj, c->d_cos, c->d_sin, c->d_meta, c->d_zero, c->d_tinypx, c->d_gemm_ws,
                    c->d_attn_ws, c->d_sentinels, c->d_pre_ws, c->d_gu, c->a1};
    for (void *b : bufs)
        if (b) (void)hipFree(b);
    if (c->h_stage) (void)hipHostFree(c->h_stage);
    if (c->stage_ev) (void)hipEventDestroy(c->stage_ev);
    for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
    delete c;
}

}  // namespace

// =========================================================================================
// C ABI
// =========================================================================================
extern "C" {

size_t vit_blob_elems(const vit_config *cfg)
{
    if (!cfg || !check_config(*cfg).empty()) return 0;
    return blob_elems_of(*cfg);
}

vit_status vit_create(const vit_weights *w, vit_ctx **out)
{
    if (!out) return fail(nullptr, VIT_E_ARG, "out is NULL");
    *out = nullptr;
    if (!w || !w->blob) return fail(nullptr, VIT_E_ARG, "weights or blob is NULL");
    const std::string why = check_config(w->cfg);
    if (!why.empty()) return fail(nullptr, VIT_E_ARG, "invalid config: " + why);
    const size_t want = blob_elems_of(w->cfg);
    if (w->blob_elems != want)
        return fail(nullptr, VIT_E_ARG, "blob has " + std::to_string(w->blob_elems) +
                                            " elements, config needs " + std::to_string(want));

    vit_ctx *c = new vit_ctx();
    c->cfg = w->cfg;
    c->D = w->cfg.hidden;
    c->H = w->cfg.heads;
    c->hd = c->D / c->H;
    c->F = w->cfg.mlp;
    c->Dl = w->cfg.out_hidden;
    c->L = w->cfg.layers;
    c->ps = w->cfg.patch;
    const int P = 3 * c->ps * c->ps;
    c->Kp = patch_gemm_k(c->ps);
    for (int i = 0; i < 3; ++i) {
        const double sd = (double)w->cfg.pix_std[i], mu = (double)w->cfg.pix_mean[i];
        c->s3[i] = (float)(1.0 / (255.0 * sd));
        c->t3[i] = (float)(-mu / sd);
    }
    auto bad = [&](vit_status st, const std::string &m) {
        g_err = m;
        destroy(c);
        return st;
    };
#define CREATE_HIP(expr)                                                                      \
    do {                                                                                      \
        hipError_t e_ = (expr);                                                               \
        if (e_ != hipSuccess) {                                                               \
            (void)hipGetLastError();                                                          \
            return bad(e_ == hipErrorOutOfMemory ? VIT_E_NOMEM : VIT_E_DEVICE,                \
                       std::string(#expr) + ": " + hipGetErrorString(e_));                    \
        }                                                                                     \
    } while (0)

    CREATE_HIP(hipGetDevice(&c->device));
    {   // the no-allocation entry point's scratch on this device, resolved at set-up
        hipError_t e_ = hipSuccess;
        if (!scratch_on_device(c->device, &e_)) {
            (void)hipGetLastError();
            return bad(VIT_E_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e_));
        }
    }
    CREATE_HIP(hipEventCreateWithFlags(&c->stage_ev, hipEventDisableTiming));
    CREATE_HIP(hipMalloc((void **)&c->d_zero, 256));
    CREATE_HIP(hipMemset(c->d_zero, 0, 256));
    CREATE_HIP(hipMalloc((void **)&c->d_tinypx, 64));
    CREATE_HIP(hipMemset(c->d_tinypx, 0, 64));
    CREATE_HIP(hipMalloc((void **)&c->d_blob, want * sizeof(bf16_t)));
    CREATE_HIP(hipMemcpy(c->d_blob, w->blob, want * sizeof(bf16_t), hipMemcpyHostToDevice));

    const size_t D = c->D, F = c->F, Dl = c->Dl;
    const bool rms = w->cfg.norm_kind == 1, swiglu = w->cfg.mlp_kind == 1;
    c->Da = w->cfg.aligner_hidden > 0 ? w->cfg.aligner_hidden : c->Dl;
    const size_t Da = c->Da;
    const uint16_t *hb = w->blob;
    size_t off = 0;
    auto take = [&](size_t n) { const size_t o = off; off += n; return o; };
    const size_t o_wpe = take(D * P), o_bpe = take(D);
    c->pe_b = c->d_blob + o_bpe;
    c->layers.resize(c->L);
    // SwiGLU: blob offsets of each layer's gate and up tensors, interleaved below
    std::vector<size_t> o_gate(c->L), o_up(c->L), o_bgate(c->L), o_bup(c->L);
    for (int l = 0; l < c->L; ++l) {
        Layer &y = c->layers[l];
        y.ln1g = c->d_blob + take(D);
        y.ln1b = rms ? nullptr : c->d_blob + take(D);
        y.wqkv = c->d_blob + take(3 * D * D);
        y.bqkv = c->d_blob + take(3 * D);
        y.wo = c->d_blob + take(D * D);
        y.bo = c->d_blob + take(D);
        y.ln2g = c->d_blob + take(D);
        y.ln2b = rms ? nullptr : c->d_blob + take(D);
        if (swiglu) {
            o_gate[l] = take(F * D);
            o_bgate[l] = take(F);
            o_up[l] = take(F * D);
            o_bup[l] = take(F);
        } else {
            y.w1 = c->d_blob + take(F * D);
            y.b1 = c->d_blob + take(F);
        }
        y.w2 = c->d_blob + take(D * F);
        y.b2 = c->d_blob + take(D);
    }
    c->lnf_g = c->d_blob + take(D);
    c->lnf_b = rms ? nullptr : c->d_blob + take(D);
    const size_t o_wproj = take(Da * 9 * D);
    c->proj_b = c->d_blob + take(Da);
    if (w->cfg.aligner_hidden > 0) {
        c->wproj2 = c->d_blob + take(Dl * Da);
        c->proj2_b = c->d_blob + take(Dl);
    }

    // SwiGLU gate and up rows interleaved in groups of 8 (the ACT_SWIGLU layout): per layer
    // [2F][D] weights, then the [2F] biases of all layers
    if (swiglu && c->L > 0) {
        const size_t per = 2 * F * D;
        CREATE_HIP(hipMalloc((void **)&c->d_gu, (per + 2 * F) * c->L * sizeof(bf16_t)));
        std::vector<uint16_t> wl(per), bl(2 * F);
        for (int l = 0; l < c->L; ++l) {
            for (size_t f = 0; f < F; ++f) {
                const size_t r = (f / 8) * 16 + f % 8;
                std::memcpy(&wl[r * D], hb + o_gate[l] + f * D, D * sizeof(uint16_t));
                std::memcpy(&wl[(r + 8) * D], hb + o_up[l] + f * D, D * sizeof(uint16_t));
                bl[r] = hb[o_bgate[l] + f];
                bl[r + 8] = hb[o_bup[l] + f];
            }
            bf16_t *dw = c->d_gu + per * l, *db = c->d_gu + per * c->L + 2 * F * l;
            CREATE_HIP(hipMemcpy(dw, wl.data(), per * sizeof(bf16_t), hipMemcpyHostToDevice));
            CREATE_HIP(hipMemcpy(db, bl.data(), 2 * F * sizeof(bf16_t), hipMemcpyHostToDevice));
            c->layers[l].w1 = dw;
            c->layers[l].b1 = db;
        }
    }

    // patch projection weight in the fused loader's K order: column (c, y, x) of the pages'
    // patch vector ([Z] "Step 1") moves to y * RP + 3 x + c (the pixel bytes of patch row y as
    // the image stores them, each row padded to RP columns); every other column is zero
    // ([Z] "Step 5": zero padding leaves the product unchanged)
    {
        const int ps = c->ps, rp = patch_segment_cols(ps);
        std::vector<uint16_t> pad(D * c->Kp, 0);
        for (size_t r = 0; r < D; ++r)
            for (int ch = 0; ch < 3; ++ch)
                for (int y = 0; y < ps; ++y)
                    for (int x = 0; x < ps; ++x)
                        pad[r * c->Kp + (size_t)y * rp + 3 * x + ch] = hb[o_wpe + r * P + (size_t)ch * ps * ps + y * ps + x];
        CREATE_HIP(hipMalloc((void **)&c->d_wpe, pad.size() * sizeof(bf16_t)));
        CREATE_HIP(hipMemcpy(c->d_wpe, pad.data(), pad.size() * sizeof(bf16_t), hipMemcpyHostToDevice));
    }
    // projector weight permuted from channel-major (c*9 + pos) to position-major (pos*D + c)
    {
        std::vector<uint16_t> perm(Da * 9 * D);
        for (size_t j = 0; j < Da; ++j) {
            const uint16_t *src = hb + o_wproj + j * 9 * D;
            uint16_t *dstp = &perm[j * 9 * D];
            for (size_t ch = 0; ch < D; ++ch)
                for (int pos = 0; pos < 9; ++pos) dstp[pos * D + ch] = src[ch * 9 + pos];
        }
        CREATE_HIP(hipMalloc((void **)&c->d_wproj, perm.size() * sizeof(bf16_t)));
        CREATE_HIP(hipMemcpy(c->d_wproj, perm.data(), perm.size() * sizeof(bf16_t), hipMemcpyHostToDevice));
    }
    // RoPE tables: cos/sin of p * f_j, f_j = base^(-2j/(hd/2)), j < hd/4 ([Z] "Step 3")
    {
        const int Q4 = c->hd / 4, half = c->hd / 2;
        std::vector<float> cs((size_t)kMaxSide * Q4), sn((size_t)kMaxSide * Q4);
        for (int pos = 0; pos < kMaxSide; ++pos)
            for (int j = 0; j < Q4; ++j) {
                const double f = std::pow((double)w->cfg.rope_base, -2.0 * j / (double)half);
                const double ang = (double)pos * f;
                cs[(size_t)pos * Q4 + j] = (float)std::cos(ang);
                sn[(size_t)pos * Q4 + j] = (float)std::sin(ang);
            }
        CREATE_HIP(hipMalloc((void **)&c->d_cos, cs.size() * sizeof(float)));
        CREATE_HIP(hipMalloc((void **)&c->d_sin, sn.size() * sizeof(float)));
        CREATE_HIP(hipMemcpy(c->d_cos, cs.data(), cs.size() * sizeof(float), hipMemcpyHostToDevice));
        CREATE_HIP(hipMemcpy(c->d_sin, sn.data(), sn.size() * sizeof(float), hipMemcpyHostToDevice));
    }
#undef CREATE_HIP
    *out = c;
    return VIT_OK;
}

void vit_destroy(vit_ctx *ctx) { destroy(ctx); }

vit_status vit_reserve(vit_ctx *ctx, int64_t max_patches)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (max_patches <= 0) {
        ctx->reserve_cap = 0;
        return VIT_OK;
    }
    ctx->reserve_cap = 0;
    // the transposed-V buffer also holds per-image padding (up to 63 columns per image); it
    // is sized here for 64 images and may still grow for batches with more images
    vit_status st = ensure_workspace(ctx, max_patches, max_patches + (int64_t)kVtAlign * 64);
    if (st != VIT_OK) return st;
    if ((st = ensure_tokens(ctx, max_patches)) != VIT_OK) return st;
    ctx->reserve_cap = max_patches;
    return VIT_OK;
}

int64_t vit_num_tokens(const vit_ctx *ctx, const vit_grid *h_grids, int32_t n_images)
{
    if (!ctx || n_images < 0 || (n_images > 0 && !h_grids)) return -1;
    int64_t m = 0;
    for (int i = 0; i < n_images; ++i) {
        if (h_grids[i].gh < 1 || h_grids[i].gw < 1) return -1;
        m += tokens_of(h_grids[i].gh, h_grids[i].gw);
    }
    return m;
}

int64_t vit_num_patches(const vit_ctx *ctx, const vit_grid *h_grids, int32_t n_images)
{
    if (!ctx || n_images < 0 || (n_images > 0 && !h_grids)) return -1;
    int64_t m = 0;
    for (int i = 0; i < n_images; ++i) {
        if (h_grids[i].gh < 1 || h_grids[i].gw < 1) return -1;
        m += (int64_t)h_grids[i].gh * h_grids[i].gw;
    }
    return m;
}

vit_status vit_encode(vit_ctx *ctx, const uint8_t *d_pixels, const vit_grid *h_grids,
                      int32_t n_images, float *d_out_rows, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    return encode_impl(ctx, d_pixels, h_grids, n_images, d_out_rows, (hipStream_t)stream,
                       kStopNone, 0, nullptr, 0);
}

vit_status vit_dump(vit_ctx *ctx, int32_t boundary, int32_t arg, const uint8_t *d_pixels,
                    const vit_grid *h_grids, int32_t n_images, void *d_dst, size_t dst_bytes,
                    void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (boundary < 0) return fail(ctx, VIT_E_ARG, "unknown dump boundary");
    return encode_impl(ctx, d_pixels, h_grids, n_images, nullptr, (hipStream_t)stream, boundary,
                       arg, d_dst, dst_bytes);
}

namespace {

vit_status layout_impl(int layout, const vit_grid *h_grids, int32_t n_images, int32_t merge, int32_t *h_types,
                       int32_t *h_src, int64_t *n_positions)
{
    if (!n_positions) return fail(nullptr, VIT_E_ARG, "n_positions is NULL");
    if (n_images < 0 || (n_images > 0 && !h_grids) || merge < 1)
        return fail(nullptr, VIT_E_ARG, "bad grids or merge");
    int64_t total = 0;
    for (int i = 0; i < n_images; ++i) {
        if (h_grids[i].gh < 1 || h_grids[i].gw < 1) return fail(nullptr, VIT_E_ARG, "bad grid");
        const int64_t mh = (h_grids[i].gh + merge - 1) / merge, mw = (h_grids[i].gw + merge - 1) / merge;
        total += span_length(layout, mh, mw);
    }
    *n_positions = total;
    if (!h_types && !h_src) return VIT_OK;
    int64_t p = 0, first = 0;
    for (int i = 0; i < n_images; ++i) {
        const int64_t mh = (h_grids[i].gh + merge - 1) / merge, mw = (h_grids[i].gw + merge - 1) / merge;
        const int64_t len = span_length(layout, mh, mw);
        for (int64_t k = 0; k < len; ++k, ++p) {
            int64_t tok;
            const int t = span_entry(layout, mh, mw, k, &tok);
            if (h_types) h_types[p] = t;
            if (h_src) h_src[p] = tok >= 0 ? (int32_t)(first + tok) : -1;
        }
        first += mh * mw;
    }
    return VIT_OK;
}

}  // namespace

vit_status vit_layout(const vit_grid *h_grids, int32_t n_images, int32_t merge, int32_t *h_types,
                      int32_t *h_src, int64_t *n_positions)
{
    return layout_impl(VIT_SPAN_V41, h_grids, n_images, merge, h_types, h_src, n_positions);
}

vit_status vit_layout_v4(const vit_grid *h_grids, int32_t n_images, int32_t merge, int32_t *h_types,
                         int32_t *h_src, int64_t *n_positions)
{
    return layout_impl(VIT_SPAN_V4, h_grids, n_images, merge, h_types, h_src, n_positions);
}

vit_status vit_set_span_layout(vit_ctx *ctx, int32_t layout)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (layout != VIT_SPAN_V41 && layout != VIT_SPAN_V4) return fail(ctx, VIT_E_ARG, "unknown span layout");
    ctx->span_layout = layout;
    return VIT_OK;
}

vit_status vit_overlay(vit_ctx *ctx, uint16_t *d_embeds, int64_t n_embed_rows,
                       const int32_t *h_rows, const float *d_rows, int64_t n_rows, int32_t hidden,
                       void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (n_rows < 0 || n_embed_rows < 0 || hidden < 1)
        return fail(ctx, VIT_E_ARG, "negative size or hidden < 1");
    if (hidden != ctx->Dl) return fail(ctx, VIT_E_ARG, "hidden does not match out_hidden");
    if (n_rows == 0) return VIT_OK;
    if (!d_embeds || !h_rows || !d_rows) return fail(ctx, VIT_E_ARG, "NULL pointer");
    std::vector<int32_t> dsts;
    dsts.reserve(n_rows);
    for (int64_t t = 0; t < n_rows; ++t) {
        const int32_t r = h_rows[t];
        if (r >= n_embed_rows) return fail(ctx, VIT_E_ARG, "placeholder row out of range");
        if (r >= 0) dsts.push_back(r);
    }
    std::sort(dsts.begin(), dsts.end());
    if (std::adjacent_find(dsts.begin(), dsts.end()) != dsts.end())
        return fail(ctx, VIT_E_ARG, "two visual rows target the same placeholder row");
    std::vector<size_t> off;
    vit_status st = upload_meta(ctx, {{h_rows, (size_t)n_rows * sizeof(int32_t)}},
                                (hipStream_t)stream, off);
    if (st != VIT_OK) return st;
    TLAUNCH(ctx, VIT_STEP_OVERLAY, (hipStream_t)stream, launch_overlay(d_embeds, d_rows, (const int32_t *)(ctx->d_meta + off[0]), n_rows,
                               hidden, (hipStream_t)stream));
    return VIT_OK;
}

vit_status vit_plan_image(int32_t height, int32_t width, int32_t patch, int32_t merge, int32_t max_tokens,
                          int64_t min_pixels, int32_t max_aspect, vit_image_plan *out)
{
    if (!out) return fail(nullptr, VIT_E_ARG, "out is NULL");
    if (height < 1 || width < 1 || height > 65536 || width > 65536 || patch < 1 || merge < 1 ||
        max_tokens < 1 || min_pixels < 0 || max_aspect < 0)
        return fail(nullptr, VIT_E_ARG, "bad image size or planning parameter");
    const double u = (double)patch * merge;
    double H1 = height, W1 = width;
    const double px = (double)height * width;
    if (px < (double)min_pixels) {   // enlarged proportionally first
        const double sc = std::sqrt((double)min_pixels / px);
        H1 *= sc;
        W1 *= sc;
    }
    if (max_aspect > 0) {            // planning aspect limited to max_aspect : 1
        if (W1 > max_aspect * H1) H1 = W1 / max_aspect;
        else if (H1 > max_aspect * W1) W1 = H1 / max_aspect;
    }
    const double a = H1 / u, b = W1 / u;
    int64_t mh = 0, mw = 0;
    if (a * b <= (double)max_tokens) {   // the image fits the budget: nearest grid
        mh = std::max<int64_t>(1, (int64_t)std::nearbyint(a));
        mw = std::max<int64_t>(1, (int64_t)std::nearbyint(b));
    }
    if (mh * mw == 0 || mh * mw > max_tokens) {   // largest grid of the image's aspect in the budget
        const double r = std::sqrt((double)max_tokens / (a * b));
        mh = std::max<int64_t>(1, (int64_t)std::floor(a * r));
        mw = std::max<int64_t>(1, (int64_t)std::floor(b * r));
        const double target = std::log(b / a);
        for (;;) {
            const bool rows_ok = (mh + 1) * mw <= max_tokens, cols_ok = mh * (mw + 1) <= max_tokens;
            if (!rows_ok && !cols_ok) break;
            const double er = rows_ok ? std::fabs(std::log((double)mw / (double)(mh + 1)) - target) : 0.0;
            const double ec = cols_ok ? std::fabs(std::log((double)(mw + 1) / (double)mh) - target) : 0.0;
            if (rows_ok && (!cols_ok || er <= ec)) ++mh;
            else ++mw;
        }
    }
    if (mh * merge * patch > 65536 || mw * merge * patch > 65536) return fail(nullptr, VIT_E_ARG, "canvas too large");
    vit_image_plan p{};
    p.gh = (int32_t)(mh * merge);
    p.gw = (int32_t)(mw * merge);
    p.canvas_h = p.gh * patch;
    p.canvas_w = p.gw * patch;
    // contain: the limiting side fills the canvas, the other is rounded (half to even)
    auto round_div = [](int64_t num, int64_t den) {
        int64_t q = num / den, r = num % den;
        if (2 * r > den || (2 * r == den && (q & 1))) ++q;
        return q;
    };
    if ((int64_t)width * p.canvas_h >= (int64_t)height * p.canvas_w) {
        p.resized_w = p.canvas_w;
        p.resized_h = (int32_t)std::max<int64_t>(1, round_div((int64_t)height * p.canvas_w, width));
    } else {
        p.resized_h = p.canvas_h;
        p.resized_w = (int32_t)std::max<int64_t>(1, round_div((int64_t)width * p.canvas_h, height));
    }
    p.off_y = (p.canvas_h - p.resized_h) / 2;
    p.off_x = (p.canvas_w - p.resized_w) / 2;
    *out = p;
    return VIT_OK;
}

vit_status vit_preprocess(vit_ctx *ctx, const uint8_t *d_src, int32_t height, int32_t width,
                          const vit_image_plan *plan, uint8_t *d_canvas, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (!plan || !d_src || !d_canvas) return fail(ctx, VIT_E_ARG, "NULL pointer");
    const vit_image_plan &p = *plan;
    if (height < 1 || width < 1 || p.gh < 1 || p.gw < 1 || p.canvas_h != p.gh * ctx->ps ||
        p.canvas_w != p.gw * ctx->ps || p.resized_h < 1 || p.resized_w < 1 || p.off_y < 0 || p.off_x < 0 ||
        p.off_y + p.resized_h > p.canvas_h || p.off_x + p.resized_w > p.canvas_w)
        return fail(ctx, VIT_E_ARG, "plan does not fit the image or the context's patch size");
    const size_t need = (size_t)height * p.resized_w * 3 * sizeof(float);
    if (need > ctx->pre_ws_bytes) {
        if (hipDeviceSynchronize() != hipSuccess) (void)hipGetLastError();
        if (ctx->d_pre_ws) (void)hipFree(ctx->d_pre_ws);
        ctx->d_pre_ws = nullptr;
        ctx->pre_ws_bytes = 0;
        if (hipMalloc((void **)&ctx->d_pre_ws, need) != hipSuccess) {
            (void)hipGetLastError();
            ctx->d_pre_ws = nullptr;
            return fail(ctx, VIT_E_NOMEM, "cannot allocate the resize scratch");
        }
        ctx->pre_ws_bytes = need;
    }
    LAUNCH(ctx, launch_preprocess(d_src, height, width, ctx->d_pre_ws, p.resized_h, p.resized_w, d_canvas,
                                  p.canvas_h, p.canvas_w, p.off_y, p.off_x, (hipStream_t)stream));
    return VIT_OK;
}

vit_status vit_set_sentinels(vit_ctx *ctx, const uint16_t *h_sentinels, int32_t hidden)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (hidden != ctx->Dl) return fail(ctx, VIT_E_ARG, "hidden does not match out_hidden");
    if (!h_sentinels) return fail(ctx, VIT_E_ARG, "NULL pointer");
    const size_t bytes = (size_t)3 * ctx->Dl * sizeof(uint16_t);
    if (!ctx->d_sentinels) {
        if (hipMalloc((void **)&ctx->d_sentinels, bytes) != hipSuccess) {
            (void)hipGetLastError();
            ctx->d_sentinels = nullptr;
            return fail(ctx, VIT_E_NOMEM, "cannot allocate the sentinel rows");
        }
    }
    HIP_TRY(ctx, hipMemcpy(ctx->d_sentinels, h_sentinels, bytes, hipMemcpyHostToDevice));
    return VIT_OK;
}

vit_status vit_assemble(vit_ctx *ctx, uint16_t *d_embeds, int64_t chunk_lo, int64_t chunk_hi,
                        int32_t hidden, const vit_grid *h_grids, int32_t n_images,
                        const int64_t *h_span_start, const float *d_rows, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (hidden != ctx->Dl) return fail(ctx, VIT_E_ARG, "hidden does not match out_hidden");
    if (chunk_lo < 0 || chunk_hi < chunk_lo || chunk_hi - chunk_lo > INT32_MAX)
        return fail(ctx, VIT_E_ARG, "bad chunk range");
    Plan p;
    vit_status st = make_plan(ctx, h_grids, n_images, p);
    if (st != VIT_OK) return st;
    if (n_images > 0 && !h_span_start) return fail(ctx, VIT_E_ARG, "NULL pointer");
    if (!ctx->d_sentinels) return fail(ctx, VIT_E_ARG, "no sentinel rows: call vit_set_sentinels first");
    // spans: START, mh x (mw IMAGE, NEWLINE), END; they must not overlap
    const int lay = ctx->span_layout;
    std::vector<std::pair<int64_t, int64_t>> spans;
    for (int i = 0; i < n_images; ++i) {
        const ImgDesc &d = p.imgs[i];
        if (h_span_start[i] < 0) return fail(ctx, VIT_E_ARG, "negative span start");
        if (lay == VIT_SPAN_V4 && h_span_start[i] % kSpanAlign)
            return fail(ctx, VIT_E_ARG, "V4 Flash spans start at multiples of 4");
        spans.push_back({h_span_start[i], span_length(lay, d.mh, d.mw)});
    }
    std::vector<std::pair<int64_t, int64_t>> sorted = spans;
    std::sort(sorted.begin(), sorted.end());
    for (size_t i = 1; i < sorted.size(); ++i)
        if (sorted[i].first < sorted[i - 1].first + sorted[i - 1].second)
            return fail(ctx, VIT_E_ARG, "image spans overlap");
    std::vector<int32_t> entries;   // (row of the chunk, source) pairs
    for (int i = 0; i < n_images; ++i) {
        const ImgDesc &d = p.imgs[i];
        const int64_t s0 = spans[i].first, len = spans[i].second;
        const int64_t lo = std::max(s0, chunk_lo), hi = std::min(s0 + len, chunk_hi);
        for (int64_t pos = lo; pos < hi; ++pos) {
            int64_t tok;
            const int t = span_entry(lay, d.mh, d.mw, pos - s0, &tok);
            if (t == VIT_TOK_PAD) continue;                 // left as the caller wrote it
            const int32_t src = t == VIT_TOK_IMAGE ? (int32_t)(d.tok_off + tok)
                                : t == VIT_TOK_START ? -1 : t == VIT_TOK_NEWLINE ? -2 : -3;
            entries.push_back((int32_t)(pos - chunk_lo));
            entries.push_back(src);
        }
    }
    if (entries.empty()) return VIT_OK;
    if (!d_embeds || !d_rows) return fail(ctx, VIT_E_ARG, "NULL pointer");
    std::vector<size_t> off;
    st = upload_meta(ctx, {{entries.data(), entries.size() * sizeof(int32_t)}}, (hipStream_t)stream, off);
    if (st != VIT_OK) return st;
    TLAUNCH(ctx, VIT_STEP_OVERLAY, (hipStream_t)stream,
            launch_assemble(d_embeds, d_rows, ctx->d_sentinels, (const int32_t *)(ctx->d_meta + off[0]),
                            (int64_t)entries.size() / 2, hidden, (hipStream_t)stream));
    return VIT_OK;
}

vit_status vit_timing_enable(vit_ctx *ctx, int32_t enable)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    ctx->timing = enable != 0;
    return VIT_OK;
}

vit_status vit_timing_read(vit_ctx *ctx, float *ms, int64_t *launches)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (ms)
        for (int k = 0; k < VIT_STEP_COUNT; ++k) ms[k] = 0.f;
    if (launches)
        for (int k = 0; k < VIT_STEP_COUNT; ++k) launches[k] = 0;
    if (!ctx->ev_marks.empty()) {
        HIP_TRY(ctx, hipEventSynchronize(ctx->ev_pool[ctx->ev_marks.back().second + 1]));
        for (auto &m : ctx->ev_marks) {
            float t = 0.f;
            HIP_TRY(ctx, hipEventElapsedTime(&t, ctx->ev_pool[m.second], ctx->ev_pool[m.second + 1]));
            if (ms) ms[m.first] += t;
            if (launches) launches[m.first] += 1;
        }
    }
    ctx->ev_marks.clear();
    ctx->ev_next = 0;
    return VIT_OK;
}

const char *vit_last_error(const vit_ctx *ctx) { return ctx ? ctx->err.c_str() : g_err.c_str(); }

// ---------------------------------------------------------------------------------------
// single-step entry points (vit_ops.h)
// ---------------------------------------------------------------------------------------
vit_status vit_op_linear(vit_ctx *ctx, const uint16_t *d_A, int64_t M, int32_t K,
                         const uint16_t *d_W, const uint16_t *d_b, int32_t N, int32_t act,
                         int32_t out_f32, void *d_out, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (M < 0 || N < 1 || K < 64 || K % 64) return fail(ctx, VIT_E_ARG, "bad M, N or K");
    if (act != VIT_ACT_NONE && act != VIT_ACT_GELU_TANH && act != VIT_ACT_GELU_ERF && act != VIT_ACT_SWIGLU)
        return fail(ctx, VIT_E_ARG, "bad act");
    if (act != VIT_ACT_NONE && out_f32) return fail(ctx, VIT_E_ARG, "fp32 output takes no activation");
    if (act == VIT_ACT_SWIGLU && N % 16) return fail(ctx, VIT_E_ARG, "SwiGLU needs N % 16 == 0");
    if (M == 0) return VIT_OK;
    if (!d_A || !d_W || !d_out) return fail(ctx, VIT_E_ARG, "NULL pointer");
    const GemmWorkspace gws = gemm_ws(ctx);
    LAUNCH(ctx, launch_linear(d_A, M, K, d_W, d_b, N, act, out_f32 != 0, d_out, &gws, (hipStream_t)stream));
    return VIT_OK;
}

vit_status vit_op_linear_noalloc(vit_ctx *ctx, const uint16_t *d_A, int64_t M, int32_t K,
                                 const uint16_t *d_W, const uint16_t *d_b, int32_t N, int32_t act,
                                 int32_t out_f32, void *d_out, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (M < 0 || N < 1 || K < 64 || K % 64) return fail(ctx, VIT_E_ARG, "bad M, N or K");
    if (act != VIT_ACT_NONE && act != VIT_ACT_GELU_TANH && act != VIT_ACT_GELU_ERF && act != VIT_ACT_SWIGLU)
        return fail(ctx, VIT_E_ARG, "bad act");
    if (act != VIT_ACT_NONE && out_f32) return fail(ctx, VIT_E_ARG, "fp32 output takes no activation");
    if (act == VIT_ACT_SWIGLU && N % 16) return fail(ctx, VIT_E_ARG, "SwiGLU needs N % 16 == 0");
    if (M == 0) return VIT_OK;
    if (!d_A || !d_W || !d_out) return fail(ctx, VIT_E_ARG, "NULL pointer");
    const size_t need = linear_workspace_bytes(M, K, N, act, out_f32 != 0);
    if (need > kNoAllocScratchBytes)
        return fail(ctx, VIT_E_ARG, "this GEMM's split-K partials need " + std::to_string(need) +
                                        " bytes, more than the " + std::to_string(kNoAllocScratchBytes) +
                                        "-byte fixed scratch of the no-allocation entry point");
    int dev = 0;
    HIP_TRY(ctx, hipGetDevice(&dev));
    hipError_t e = hipSuccess;
    float *part = scratch_on_device(dev, &e);   // first call on a device resolves it here
    if (!part) return fail(ctx, VIT_E_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    const GemmWorkspace gws{part, kNoAllocScratchBytes};
    LAUNCH(ctx, launch_linear(d_A, M, K, d_W, d_b, N, act, out_f32 != 0, d_out, &gws, (hipStream_t)stream));
    return VIT_OK;
}

vit_status vit_op_linear_residual(vit_ctx *ctx, const uint16_t *d_A, int64_t M, int32_t K, const uint16_t *d_W,
                                  const uint16_t *d_b, int32_t N, uint16_t *d_x, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (M < 0 || N < 1 || K < 64 || K % 64) return fail(ctx, VIT_E_ARG, "bad M, N or K");
    if (M == 0) return VIT_OK;
    if (!d_A || !d_W || !d_x) return fail(ctx, VIT_E_ARG, "NULL pointer");
    const uintptr_t a0 = (uintptr_t)d_A, a1 = a0 + (uintptr_t)M * K * 2, x0 = (uintptr_t)d_x,
                    x1 = x0 + (uintptr_t)M * N * 2;
    if (a0 < x1 && x0 < a1) return fail(ctx, VIT_E_ARG, "A overlaps x");
    const GemmWorkspace gws = gemm_ws(ctx);
    LAUNCH(ctx, launch_linear_residual(d_A, M, K, d_W, d_b, N, d_x, &gws, (hipStream_t)stream));
    return VIT_OK;
}

vit_status vit_op_layernorm(vit_ctx *ctx, const uint16_t *d_x, const uint16_t *d_delta,
                            uint16_t *d_xout, int64_t M, int32_t D, const uint16_t *d_g,
                            const uint16_t *d_b, float eps, uint16_t *d_out, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (M < 0 || !supported_hidden(D)) return fail(ctx, VIT_E_ARG, "bad M or D");
    if (M == 0) return VIT_OK;
    if (!d_x || !d_g || !d_b || !d_out || (d_delta && !d_xout)) return fail(ctx, VIT_E_ARG, "NULL pointer");
    LAUNCH(ctx, launch_layernorm(d_x, d_delta, d_xout, M, D, d_g, d_b, eps, false, d_out, (hipStream_t)stream));
    return VIT_OK;
}

vit_status vit_op_rmsnorm(vit_ctx *ctx, const uint16_t *d_x, const uint16_t *d_delta, uint16_t *d_xout, int64_t M,
                          int32_t D, const uint16_t *d_g, float eps, uint16_t *d_out, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (M < 0 || !supported_hidden(D)) return fail(ctx, VIT_E_ARG, "bad M or D");
    if (M == 0) return VIT_OK;
    if (!d_x || !d_g || !d_out || (d_delta && !d_xout)) return fail(ctx, VIT_E_ARG, "NULL pointer");
    LAUNCH(ctx, launch_layernorm(d_x, d_delta, d_xout, M, D, d_g, nullptr, eps, true, d_out, (hipStream_t)stream));
    return VIT_OK;
}

int64_t vit_vt_stride(const vit_grid *h_grids, int32_t n_images)
{
    if (n_images < 0 || (n_images > 0 && !h_grids)) return -1;
    int64_t cols = 0;
    for (int i = 0; i < n_images; ++i) {
        if (h_grids[i].gh < 1 || h_grids[i].gw < 1) return -1;
        cols += ceil_div((int64_t)h_grids[i].gh * h_grids[i].gw, kVtAlign) * kVtAlign;
    }
    return cols;
}

vit_status vit_op_rope(vit_ctx *ctx, uint16_t *d_qkv, uint16_t *d_vt, const vit_grid *h_grids,
                       int32_t n_images, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    Plan p;
    vit_status st = make_plan(ctx, h_grids, n_images, p);
    if (st != VIT_OK) return st;
    if (p.N == 0) return VIT_OK;
    if (!d_qkv || !d_vt) return fail(ctx, VIT_E_ARG, "NULL pointer");
    DevPlan dp{};
    if ((st = stage_plan(ctx, p, (hipStream_t)stream, dp)) != VIT_OK) return st;
    LAUNCH(ctx, launch_rope(d_qkv, d_vt, p.vt_cols, dp.rope, (int)p.rope.size(), dp.imgs, ctx->D,
                            ctx->H, ctx->d_cos, ctx->d_sin, (hipStream_t)stream));
    return VIT_OK;
}

vit_status vit_op_qkv_rope(vit_ctx *ctx, const uint16_t *d_x, const uint16_t *d_W, const uint16_t *d_b,
                           const vit_grid *h_grids, int32_t n_images, uint16_t *d_qkv, uint16_t *d_vt,
                           int32_t store_v, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    Plan p;
    vit_status st = make_plan(ctx, h_grids, n_images, p);
    if (st != VIT_OK) return st;
    if (p.N == 0) return VIT_OK;
    if (!d_x || !d_W || !d_qkv || !d_vt) return fail(ctx, VIT_E_ARG, "NULL pointer");
    DevPlan dp{};
    if ((st = stage_plan(ctx, p, (hipStream_t)stream, dp)) != VIT_OK) return st;
    const int ni = (int)p.imgs.size();
    LAUNCH(ctx, launch_vt_tail_zero(d_vt, p.vt_cols, dp.imgs, ni, ctx->D, (hipStream_t)stream));
    LAUNCH(ctx, launch_qkv_rope(d_x, p.N, ctx->D, ctx->H, d_W, d_b, d_qkv, d_vt, p.vt_cols, dp.imgs, ni,
                                ctx->d_cos, ctx->d_sin, store_v != 0, (hipStream_t)stream));
    return VIT_OK;
}

vit_status vit_op_attention(vit_ctx *ctx, const uint16_t *d_qkv, const uint16_t *d_vt,
                            const vit_grid *h_grids, int32_t n_images, uint16_t *d_o, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    Plan p;
    vit_status st = make_plan(ctx, h_grids, n_images, p);
    if (st != VIT_OK) return st;
    if (p.N == 0) return VIT_OK;
    if (!d_qkv || !d_vt || !d_o) return fail(ctx, VIT_E_ARG, "NULL pointer");
    const AttnSplit asp = attn_split(ctx, p);
    DevPlan dp{};
    if ((st = stage_plan(ctx, p, (hipStream_t)stream, dp)) != VIT_OK) return st;
    LAUNCH(ctx, launch_attention(d_qkv, d_vt, p.vt_cols, d_o, dp.attn, (int)p.attn.size(), dp.imgs,
                                 ctx->D, ctx->H, asp, (hipStream_t)stream));
    LAUNCH(ctx, launch_attention_merge(d_o, dp.attn, (int)p.attn.size(), dp.imgs, ctx->D, ctx->H, asp,
                                       (hipStream_t)stream));
    return VIT_OK;
}

vit_status vit_set_attention_split(vit_ctx *ctx, int32_t n)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    if (n < 0 || n > 4) return fail(ctx, VIT_E_ARG, "attention key slices must be 0 (automatic) or 1..4");
    ctx->attn_split_fixed = n;
    return VIT_OK;
}

vit_status vit_op_merge_project(vit_ctx *ctx, const uint16_t *d_y, const vit_grid *h_grids,
                                int32_t n_images, float *d_out, void *stream)
{
    if (!ctx) return fail(nullptr, VIT_E_ARG, "ctx is NULL");
    Plan p;
    vit_status st = make_plan(ctx, h_grids, n_images, p);
    if (st != VIT_OK) return st;
    if (p.N == 0) return VIT_OK;
    if (!d_y || !d_out) return fail(ctx, VIT_E_ARG, "NULL pointer");
    DevPlan dp{};
    if ((st = stage_plan(ctx, p, (hipStream_t)stream, dp)) != VIT_OK) return st;
    const GemmWorkspace gws = gemm_ws(ctx);
    return run_aligner(ctx, d_y, dp.imgs, (int)p.imgs.size(), p.M, d_out, &gws, (hipStream_t)stream);
}

}  // extern "C"
