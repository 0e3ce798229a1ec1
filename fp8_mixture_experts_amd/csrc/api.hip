// Host side of the C ABI declared in include/mega_moe.h: argument checks, the
// per-call plan, workspace layout and the launches of the three kernel groups
// (dispatch, persistent expert kernel, combine) on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "mega_moe.h"
#include "moe_args.h"
#include "schedule.h"

namespace mega_moe {
void launch_dispatch(const MoeArgs& a, int gather_blocks, hipStream_t stream);
int launch_expert_ffn(const MoeArgs& a, int num_cus, hipStream_t stream);
void launch_combine(const MoeArgs& a, hipStream_t stream);
hipError_t probe_xcds(uint32_t* word, int num_cus, uint32_t* seen);
void launch_clear_words(uint32_t* p, int n, hipStream_t stream);
void launch_transform_w1(const uint8_t* w1, const float* sf, uint8_t* out, float* out_sf, int E,
                         int N, int H, hipStream_t stream);
}  // namespace mega_moe

using namespace mega_moe;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return MEGA_MOE_OK;
}

int64_t align_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Sizes that depend only on the configuration.
struct Layout {
    int64_t R_max, P_cap, PB_cap, chunks_max;
    int64_t off[19];
    int64_t total;
};

enum {
    L_COUNTS, L_OFFSETS, L_PBREC, L_SLOTMAP, L_SRC, L_POOLW, L_CHIST, L_CBASE,
    L_L1ACTS, L_L1SF, L_L1W, L_L2ACTS, L_L2SF, L_COMB, L_READY, L_XCDINFO, L_CTRL,
    L_COUNT
};

// 256-column tiles: both N extents must split into them, and the 32-row
// instance has none (its rows do not divide over eight waves).
bool wide_tiles_fit(const mega_moe_config& c) {
    return (2 * c.intermediate) % 256 == 0 && c.hidden % 256 == 0 && c.block_m != 32;
}

int check_config(const mega_moe_config* c) {
    if (!c) return fail(MEGA_MOE_ERR_INVALID_ARG, "config is NULL");
    if (c->num_experts < 1 || c->num_experts > MAX_EXPERTS)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "num_experts must be in [1, %d], got %d", MAX_EXPERTS,
                    c->num_experts);
    if (c->hidden <= 0 || c->hidden % 128)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "hidden must be a positive multiple of 128, got %d",
                    c->hidden);
    if (c->intermediate <= 0 || c->intermediate % 128)
        return fail(MEGA_MOE_ERR_INVALID_ARG,
                    "intermediate must be a positive multiple of 128, got %d", c->intermediate);
    if (c->hidden > 8192 || c->intermediate > 4096)
        return fail(MEGA_MOE_ERR_UNSUPPORTED,
                    "built for hidden <= 8192 and intermediate <= 4096 (got %d, %d)", c->hidden,
                    c->intermediate);
    if (c->num_topk < 1) return fail(MEGA_MOE_ERR_INVALID_ARG, "num_topk must be >= 1");
    if (c->max_tokens < 0) return fail(MEGA_MOE_ERR_INVALID_ARG, "max_tokens must be >= 0");
    if ((int64_t)c->max_tokens * c->num_topk > (int64_t)1 << 30)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "max_tokens * num_topk too large");
    if (!(c->activation_clamp > 0))        // also rejects NaN
        return fail(MEGA_MOE_ERR_INVALID_ARG, "activation_clamp must be > 0 (+inf: no clamp)");
    if (c->fast_math != 0 && c->fast_math != 1)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "fast_math must be 0 or 1");
    if (c->block_m != 0 && c->block_m != 32 && c->block_m != 64 && c->block_m != 128)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "block_m must be 0, 32, 64 or 128");
    if (c->l2_n_major < -1 || c->l2_n_major > 1)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "l2_n_major must be -1, 0 or 1");
    if (c->block_n != 0 && c->block_n != 128 && c->block_n != 256)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "block_n must be 0, 128 or 256");
    if (c->block_n == 256 && !wide_tiles_fit(*c))
        return fail(MEGA_MOE_ERR_INVALID_ARG,
                    "block_n 256 needs 2*intermediate and hidden multiples of 256 and block_m != 32");
    if (c->split_l2_cus < 0 || c->split_l2_cus > 31)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "split_l2_cus must be in [0, 31], got %d",
                    c->split_l2_cus);
    if (c->keep_pool != 0 && c->keep_pool != 1)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "keep_pool must be 0 or 1");
    if (c->split_l2_xcds < 0 || c->split_l2_xcds >= MAX_XCD)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "split_l2_xcds must be in [0, %d), got %d", MAX_XCD,
                    c->split_l2_xcds);
    if (c->split_l2_xcds > 0 && c->split_l2_cus > 0)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "split_l2_cus and split_l2_xcds exclude each other");
    // the expert kernel addresses rows of x with 32-bit byte offsets
    if ((int64_t)c->max_tokens * c->hidden > ((int64_t)1 << 31) - 2 * (int64_t)c->hidden)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "max_tokens * hidden must stay below 2^31");
    return MEGA_MOE_OK;
}

Layout make_layout(const mega_moe_config& c) {
    Layout L{};
    const int64_t E = c.num_experts, H = c.hidden, I = c.intermediate;
    L.R_max = (int64_t)c.max_tokens * c.num_topk;
    // sum over experts of align_up(count, 128) <= R + 127 E
    L.P_cap = align_up(L.R_max + (POOL_ALIGN - 1) * E, POOL_ALIGN);
    L.PB_cap = L.P_cap / 32;           // pool blocks at the smallest BLOCK_M
    L.chunks_max = (L.R_max + DISPATCH_CHUNK - 1) / DISPATCH_CHUNK;
    if (L.chunks_max < 1) L.chunks_max = 1;
    int64_t sz[L_COUNT];
    sz[L_COUNTS] = E * 4;
    sz[L_OFFSETS] = (E + 1) * 4;
    sz[L_PBREC] = L.PB_cap * 16;
    sz[L_SLOTMAP] = L.R_max * 4;
    sz[L_SRC] = L.P_cap * 4;
    sz[L_POOLW] = L.P_cap * 4;
    sz[L_CHIST] = L.chunks_max * E * 4;
    sz[L_CBASE] = L.chunks_max * E * 4;
    // the pool copies exist only when the configuration keeps the pool
    const int64_t pool_rows = c.keep_pool ? L.P_cap : 0;
    sz[L_L1ACTS] = pool_rows * H;
    sz[L_L1SF] = (H / 128) * L.P_cap * 4;   // also the 128-row tiles' pool-ordered scales
    sz[L_L1W] = pool_rows * 4;
    sz[L_L2ACTS] = L.P_cap * I;
    sz[L_L2SF] = (I / 64) * L.P_cap * 4;
    sz[L_COMB] = L.R_max * H * 2;
    sz[L_READY] = L.PB_cap * 4;
    sz[L_XCDINFO] = 2 * MAX_XCD * 4;
    sz[L_CTRL] = sizeof(MoeCtrl);
    int64_t o = 0;
    for (int i = 0; i < L_COUNT; ++i) {
        L.off[i] = o;
        o = align_up(o + sz[i], 256);
    }
    L.total = o;
    return L;
}

// BLOCK_M tiers by expected routes per expert, as in the SM90 design (13.1),
// with the thresholds of this kernel on MI355X: a tile streams its weight
// block once whatever its row count, and 32-row tiles never beat 64-row ones,
// while 128-row tiles win from about 50 expected routes per expert on.
constexpr float TIER_64_MAX = 50.5f;

void plan(const mega_moe_config& c, int32_t T, mega_moe_plan_info* p) {
    // expected routes per expert on one GPU (SM90 design 13.1 with one rank)
    const float expected = float(T) * float(c.num_topk) / float(c.num_experts);
    int bm;
    if (c.block_m) bm = c.block_m;
    else bm = expected <= TIER_64_MAX ? 64 : 128;
    int nm = c.l2_n_major;
    if (nm < 0) nm = expected >= 256.0f ? 1 : 0;   // SM90 design 12.2
    // 64-row tiles run 256 columns wide when H splits into them (2I always
    // does) (one eight-wave workgroup per CU, half the activation re-reads; measured
    // 2-5% faster across the 64-row tier on MI355X); 128-row tiles keep 128
    // columns (equal or slower at 256)
    int bn = c.block_n ? c.block_n : (bm == 64 && c.hidden % 256 == 0 ? 256 : 128);
    if (bm == 32) bn = 128;
    p->expected_tokens_per_expert = expected;
    p->block_m = bm;
    p->l2_n_major = nm;
    p->block_n = bn;
    p->l1_n_blocks = 2 * c.intermediate / bn;
    p->l2_n_blocks = c.hidden / bn;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// The argument block's sizes and options for cfg and its workspace pointers
// for layout L placed at w.
void bind_workspace(MoeArgs& a, const mega_moe_config& cfg, const Layout& L, uint8_t* w,
                    int n_xcd) {
    std::memset(&a, 0, sizeof a);
    a.H = cfg.hidden;
    a.I = cfg.intermediate;
    a.E = cfg.num_experts;
    a.k = cfg.num_topk;
    a.P_cap = L.P_cap;
    a.wait_spin_limit = 1u << 20;
    a.act_clamp = cfg.activation_clamp;
    a.fast_math = cfg.fast_math;
    a.n_xcd = n_xcd;
    a.counts = (int32_t*)(w + L.off[L_COUNTS]);
    a.offsets = (int32_t*)(w + L.off[L_OFFSETS]);
    a.pb_rec = (int32_t*)(w + L.off[L_PBREC]);
    a.slot_map = (int32_t*)(w + L.off[L_SLOTMAP]);
    a.src = (int32_t*)(w + L.off[L_SRC]);
    a.pool_w = (float*)(w + L.off[L_POOLW]);
    a.chunk_hist = (int32_t*)(w + L.off[L_CHIST]);
    a.chunk_base = (int32_t*)(w + L.off[L_CBASE]);
    a.l1_acts = w + L.off[L_L1ACTS];
    a.l1_sf = (float*)(w + L.off[L_L1SF]);
    a.l1_w = (float*)(w + L.off[L_L1W]);
    a.l2_acts = w + L.off[L_L2ACTS];
    a.l2_sf = (float*)(w + L.off[L_L2SF]);
    a.comb = (uint16_t*)(w + L.off[L_COMB]);
    a.ready = (uint32_t*)(w + L.off[L_READY]);
    a.xcd_info = (int32_t*)(w + L.off[L_XCDINFO]);
    a.ctrl = (MoeCtrl*)(w + L.off[L_CTRL]);
}

// XCDs (accelerator dies, each with its own L2) of device dev.  The expert
// kernel keeps one work queue per XCD so that the L1 tiles of a pool block
// and the L2 tiles that read their output run on one XCD and meet in its L2
// without any cache write-back; that needs the device's XCD count, and its
// compute units must split evenly over them.
int xcd_count(int dev, int num_cus, int* out) {
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev);
    if (e != hipSuccess)
        return fail(MEGA_MOE_ERR_UNSUPPORTED, "XCD count of device %d unknown: %s", dev,
                    hipGetErrorString(e));
    const int rc = mega_moe_check_xcd_layout(n, num_cus, 0);
    if (rc) return rc;
    *out = n;
    return MEGA_MOE_OK;
}

}  // namespace

struct mega_moe_handle {
    mega_moe_config cfg;
    Layout L;
    int device;
    int num_cus;
    int n_xcd;
    uint8_t* ws;
    int32_t last_T;
    MoeArgs base;   // workspace pointers and sizes filled at create
    // optional event timing of the kernel groups (4 events per call)
    std::vector<hipEvent_t> prof_events;
    int32_t prof_max = 0, prof_used = 0;
    // split phases: streams of the L1 and L2 kernels, the CUs' worth of
    // workgroups each gets, and the fork / join events
    hipStream_t split_stream[2] = {nullptr, nullptr};
    int split_cus[2] = {0, 0};
    hipEvent_t split_event[3] = {nullptr, nullptr, nullptr};
};

namespace {
void prof_release(mega_moe_handle* h) {
    for (hipEvent_t ev : h->prof_events) hipEventDestroy(ev);
    h->prof_events.clear();
    h->prof_max = h->prof_used = 0;
}

hipEvent_t prof_event(mega_moe_handle* h, int call, int which) {
    if (call < 0) return nullptr;
    return h->prof_events[(size_t)call * 4 + which];
}

void split_release(mega_moe_handle* h) {
    for (hipStream_t& st : h->split_stream)
        if (st) { hipStreamDestroy(st); st = nullptr; }
    for (hipEvent_t& ev : h->split_event)
        if (ev) { hipEventDestroy(ev); ev = nullptr; }
    h->split_cus[0] = h->split_cus[1] = 0;
}

// Sets up the split phases: two streams of their own for the L1 and L2
// kernels, forked from and joined into the caller's stream with events.  The
// two kernels get disjoint workgroup budgets that together fill the device
// (two workgroups per CU): `l2` CUs' worth per XCD for the L2 kernel, the rest
// for L1, so both are resident together whichever starts first.  Both grids
// are multiples of the XCD count, and workgroups are dealt to the XCDs in
// turn, so every XCD runs workgroups of both kernels and each takes only its
// own XCD's tiles, as in the fused kernel.
int split_setup(mega_moe_handle* h, int l2) {
    const int nx = h->base.n_xcd;
    const int per_xcd = h->num_cus / nx;
    if (l2 >= per_xcd)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "split_l2_cus %d leaves no L1 CU on an XCD of %d CUs", l2,
                    per_xcd);
    h->split_cus[0] = (per_xcd - l2) * nx;
    h->split_cus[1] = l2 * nx;
    hipError_t e = hipSuccess;
    for (int i = 0; i < 2 && e == hipSuccess; ++i)
        e = hipStreamCreateWithFlags(&h->split_stream[i], hipStreamNonBlocking);
    for (int i = 0; i < 3 && e == hipSuccess; ++i)
        e = hipEventCreateWithFlags(&h->split_event[i], hipEventDisableTiming);
    if (e != hipSuccess) {
        split_release(h);
        return fail(MEGA_MOE_ERR_HIP, "split streams: %s", hipGetErrorString(e));
    }
    return MEGA_MOE_OK;
}

// Sets up the split phases on disjoint XCD sets.  One persistent launch
// fills the device as usual; the workgroups of XCDs [0, n_xcd - l2_xcds) take
// only L1 tiles and those of the other XCDs only L2 tiles, so the two phases
// run on disjoint sets of compute units (the partition is fixed by the
// hardware's XCC_ID, no CU mask).  The dispatch gives the pool blocks to the
// L1 XCDs only, every pool block's output is written back through memory for
// the L2 XCDs, and an L2 workgroup only ever waits for L1 workgroups of other
// XCDs, which never wait: no residency assumption beyond one workgroup per XCD.
int split_setup_xcds(mega_moe_handle* h, int l2_xcds) {
    const int nx = h->base.n_xcd;
    if (l2_xcds >= nx)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "split_l2_xcds %d leaves no L1 XCD of %d", l2_xcds, nx);
    h->base.phase = PHASE_XCD_SPLIT + nx - l2_xcds;
    return MEGA_MOE_OK;
}
}  // namespace

extern "C" {

const char* mega_moe_last_error(void) { return g_last_error.c_str(); }

int mega_moe_check_xcd_layout(int32_t num_xcds, int32_t num_cus, uint32_t seen_ids) {
    if (num_xcds < 1 || num_xcds > MAX_XCD || num_cus < 1 || num_cus % num_xcds != 0)
        return fail(MEGA_MOE_ERR_UNSUPPORTED,
                    "device reports %d XCDs for %d compute units; the expert kernel needs 1..%d "
                    "XCDs with the same number of compute units each", num_xcds, num_cus, MAX_XCD);
    if (seen_ids == 0) return ok();
    // the kernel takes XCD id % num_xcds as its queue: the ids must give
    // num_xcds distinct queues
    uint32_t queues = 0;
    for (int i = 0; i < 32; ++i)
        if (seen_ids >> i & 1u) queues |= 1u << (i % num_xcds);
    if (__builtin_popcount(seen_ids) != num_xcds || __builtin_popcount(queues) != num_xcds)
        return fail(MEGA_MOE_ERR_UNSUPPORTED,
                    "workgroups report the XCD ids of mask %#x on a device of %d XCDs: the "
                    "L1 -> L2 handoff needs one work queue per XCD", seen_ids, num_xcds);
    return ok();
}

int32_t mega_moe_token_alignment(void) { return POOL_ALIGN; }

int64_t mega_moe_workspace_bytes(const mega_moe_config* cfg) {
    if (check_config(cfg) != MEGA_MOE_OK) return -1;
    return make_layout(*cfg).total;
}

int mega_moe_plan(const mega_moe_config* cfg, int32_t num_tokens, mega_moe_plan_info* out) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!out) return fail(MEGA_MOE_ERR_INVALID_ARG, "out is NULL");
    if (num_tokens < 0) return fail(MEGA_MOE_ERR_INVALID_ARG, "num_tokens < 0");
    plan(*cfg, num_tokens, out);
    return ok();
}

int mega_moe_tile_order(const mega_moe_plan_info* plan, int32_t num_experts,
                        const int32_t* block_start, int32_t n_xcd, int32_t phase,
                        int32_t* pb_out, int32_t* nb_out) {
    if (!plan || !block_start) return fail(MEGA_MOE_ERR_INVALID_ARG, "plan or block_start is NULL");
    if (plan->block_m != 32 && plan->block_m != 64 && plan->block_m != 128)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "plan block_m %d is not 32, 64 or 128", plan->block_m);
    if (num_experts < 1) return fail(MEGA_MOE_ERR_INVALID_ARG, "num_experts < 1");
    if (block_start[0] != 0) return fail(MEGA_MOE_ERR_INVALID_ARG, "block_start[0] != 0");
    for (int e = 0; e < num_experts; ++e)
        if (block_start[e + 1] < block_start[e])
            return fail(MEGA_MOE_ERR_INVALID_ARG, "block_start decreases at expert %d", e);
    if (n_xcd < 1 || n_xcd > MAX_XCD)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "n_xcd must be in [1, %d]", MAX_XCD);
    if (phase != 1 && phase != 2) return fail(MEGA_MOE_ERR_INVALID_ARG, "phase must be 1 or 2");
    const int nbs = phase == 1 ? plan->l1_n_blocks : plan->l2_n_blocks;
    if (nbs < 1) return fail(MEGA_MOE_ERR_INVALID_ARG, "plan has no N blocks for phase %d", phase);
    const int total_mb = block_start[num_experts];
    if (total_mb > 0 && (!pb_out || !nb_out))
        return fail(MEGA_MOE_ERR_INVALID_ARG, "an output array is NULL");
    std::vector<int> expert(total_mb);
    for (int e = 0; e < num_experts; ++e)
        for (int p = block_start[e]; p < block_start[e + 1]; ++p) expert[p] = e;
    const auto expert_of = [&](int p) { return expert[p]; };
    const auto start_of = [&](int e) { return (int)block_start[e]; };
    const int G = xcd_group_for(plan->block_m);
    int64_t i = 0;
    for (int x = 0; x < n_xcd; ++x) {
        int lo, cnt;
        xcd_range(total_mb, n_xcd, x, lo, cnt);
        for (int u = 0; u < cnt * nbs; ++u, ++i) {
            int pb, nb;
            tile_coords(u, lo, cnt, nbs, G, plan->l2_n_major != 0, expert_of, start_of, pb, nb);
            pb_out[i] = pb;
            nb_out[i] = nb;
        }
    }
    return ok();
}

int mega_moe_create(const mega_moe_config* cfg, mega_moe_handle** out) {
    if (!out) return fail(MEGA_MOE_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    int rc = check_config(cfg);
    if (rc) return rc;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MEGA_MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
        return fail(MEGA_MOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(MEGA_MOE_ERR_UNSUPPORTED, "device %d is %s, this library is built for gfx950",
                    dev, prop.gcnArchName);
    int n_xcd = 0;
    rc = xcd_count(dev, prop.multiProcessorCount, &n_xcd);
    if (rc) return rc;
    auto* h = new mega_moe_handle{};
    h->cfg = *cfg;
    h->L = make_layout(*cfg);
    h->device = dev;
    h->num_cus = prop.multiProcessorCount;
    h->n_xcd = n_xcd;
    e = hipMalloc((void**)&h->ws, h->L.total);
    if (e != hipSuccess) {
        const long long bytes = (long long)h->L.total;
        delete h;
        return fail(MEGA_MOE_ERR_OUT_OF_MEMORY, "hipMalloc(%lld): %s", bytes, hipGetErrorString(e));
    }
    e = hipMemset(h->ws, 0, h->L.total);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        hipFree(h->ws);
        delete h;
        return fail(MEGA_MOE_ERR_HIP, "workspace clear: %s", hipGetErrorString(e));
    }
    // the expert kernel's L1 -> L2 handoff relies on every workgroup reading
    // its own XCD from the hardware: check that the device's workgroups report
    // exactly n_xcd distinct XCDs (the control record serves as the probe's word)
    uint32_t seen = 0;
    e = probe_xcds(reinterpret_cast<uint32_t*>(h->ws + h->L.off[L_CTRL]), h->num_cus, &seen);
    if (e == hipSuccess) e = hipMemset(h->ws + h->L.off[L_CTRL], 0, sizeof(MoeCtrl));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        hipFree(h->ws);
        delete h;
        return fail(MEGA_MOE_ERR_HIP, "XCD probe: %s", hipGetErrorString(e));
    }
    rc = mega_moe_check_xcd_layout(n_xcd, h->num_cus, seen);
    if (rc) {
        const std::string msg = g_last_error;
        hipFree(h->ws);
        delete h;
        return fail(rc, "%s", msg.c_str());
    }
    bind_workspace(h->base, *cfg, h->L, h->ws, h->n_xcd);
    h->last_T = 0;
    if (cfg->split_l2_cus > 0 || cfg->split_l2_xcds > 0) {
        rc = cfg->split_l2_cus > 0 ? split_setup(h, cfg->split_l2_cus)
                                   : split_setup_xcds(h, cfg->split_l2_xcds);
        if (rc) {
            const std::string msg = g_last_error;
            hipFree(h->ws);
            delete h;
            return fail(rc, "%s", msg.c_str());
        }
    }
    *out = h;
    return ok();
}

int mega_moe_destroy(mega_moe_handle* h) {
    if (!h) return ok();
    prof_release(h);
    split_release(h);
    hipError_t e = hipFree(h->ws);
    delete h;
    if (e != hipSuccess) return fail(MEGA_MOE_ERR_HIP, "hipFree: %s", hipGetErrorString(e));
    return ok();
}

// Weights of one forward call, in either format.
struct WeightArgs {
    int fmt;                      // W_FP8_ARGS or W_MXFP4_ARGS
    const uint8_t* w1;
    const float* w1_sf;
    const uint8_t* w1_e8;
    const uint8_t* w2;
    const float* w2_sf;
    const uint8_t* w2_e8;
};
constexpr int W_FP8_ARGS = 0, W_MXFP4_ARGS = 1;

// Pointer checks of a forward call (T > 0).
static int check_tensors(const uint8_t* x, const float* x_sf, const int32_t* topk_idx,
                         const float* topk_weights, const WeightArgs& w, const uint16_t* y) {
    const bool mx = w.fmt == W_MXFP4_ARGS;
    const void* wsc1 = mx ? (const void*)w.w1_e8 : (const void*)w.w1_sf;
    const void* wsc2 = mx ? (const void*)w.w2_e8 : (const void*)w.w2_sf;
    if (!x || !x_sf || !topk_idx || !topk_weights || !w.w1 || !wsc1 || !w.w2 || !wsc2 || !y)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "a tensor pointer is NULL");
    if (!aligned(x, 16) || !aligned(w.w1, 16) || !aligned(w.w2, 16) || !aligned(y, 16))
        return fail(MEGA_MOE_ERR_INVALID_ARG, "x, w1, w2 and y must be 16-byte aligned");
    if (!aligned(x_sf, 4) || !aligned(topk_idx, 4) || !aligned(topk_weights, 4) ||
        !aligned(wsc1, 4) || !aligned(wsc2, 4))
        return fail(MEGA_MOE_ERR_INVALID_ARG, "scale, index and weight arrays must be 4-byte aligned");
    return MEGA_MOE_OK;
}

// The argument block of one call: the plan for T tokens and the tensors.
static void call_args(MoeArgs& a, const mega_moe_config& cfg, int32_t T, const uint8_t* x,
                      const float* x_sf, const int32_t* topk_idx, const float* topk_weights,
                      const WeightArgs& w, uint16_t* y) {
    const bool mx = w.fmt == W_MXFP4_ARGS;
    mega_moe_plan_info p;
    plan(cfg, T, &p);
    if (mx) {
        // MXFP4 weights run on 128-column tiles only
        p.block_n = 128;
        p.l1_n_blocks = 2 * cfg.intermediate / 128;
        p.l2_n_blocks = cfg.hidden / 128;
    }
    a.T = T;
    a.R = T * cfg.num_topk;
    a.block_m = p.block_m;
    a.block_n = p.block_n;
    a.nb1 = p.l1_n_blocks;
    a.nb2 = p.l2_n_blocks;
    a.n_major = p.l2_n_major;
    // cross-XCD tail balancing pays with the large batches of the N-major schedule
    a.steal = p.l2_n_major;
    a.merge_tail = merge_tail_for(mx, p.block_m, p.block_n);
    a.xcd_group = xcd_group_for(p.block_m);
    a.num_chunks = (a.R + DISPATCH_CHUNK - 1) / DISPATCH_CHUNK;
    a.x = x;
    a.x_sf = x_sf;
    a.topk_idx = topk_idx;
    a.topk_w = topk_weights;
    a.w_fmt = mx ? 1 : 0;
    a.w1 = w.w1;
    a.w1_sf = w.w1_sf;
    a.w1_e8 = w.w1_e8;
    a.w2 = w.w2;
    a.w2_sf = w.w2_sf;
    a.w2_e8 = w.w2_e8;
    a.y = y;
}

static int forward_impl(mega_moe_handle* h, int32_t T, const uint8_t* x, const float* x_sf,
                        const int32_t* topk_idx, const float* topk_weights, const WeightArgs& w,
                        uint16_t* y, void* stream_v) {
    if (!h) return fail(MEGA_MOE_ERR_INVALID_ARG, "handle is NULL");
    if (T < 0 || T > h->cfg.max_tokens)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "num_tokens %d outside [0, max_tokens=%d]", T,
                    h->cfg.max_tokens);
    h->last_T = T;
    if (T == 0) return ok();
    int rc = check_tensors(x, x_sf, topk_idx, topk_weights, w, y);
    if (rc) return rc;
    hipStream_t stream = (hipStream_t)stream_v;
    MoeArgs a = h->base;
    call_args(a, h->cfg, T, x, x_sf, topk_idx, topk_weights, w, y);
    const int gather_blocks = h->cfg.keep_pool ? (a.R < 16384 ? a.R : 16384) : 0;
    const int call = h->prof_used < h->prof_max ? h->prof_used++ : -1;
    if (call >= 0) hipEventRecord(prof_event(h, call, 0), stream);
    launch_dispatch(a, gather_blocks, stream);
    if (call >= 0) hipEventRecord(prof_event(h, call, 1), stream);
    if (h->split_stream[0]) {
        // the L1 and L2 tiles as two concurrent kernels with disjoint workgroup
        // budgets, forked from and joined back into the caller's stream (the
        // split on disjoint XCD sets runs in the one launch below: its
        // arguments carry the XCD roles)
        hipEventRecord(h->split_event[0], stream);
        for (int i = 0; i < 2; ++i) {
            hipStreamWaitEvent(h->split_stream[i], h->split_event[0], 0);
            MoeArgs ai = a;
            ai.phase = i + 1;
            launch_expert_ffn(ai, h->split_cus[i], h->split_stream[i]);
            hipEventRecord(h->split_event[1 + i], h->split_stream[i]);
        }
        hipStreamWaitEvent(stream, h->split_event[1], 0);
        hipStreamWaitEvent(stream, h->split_event[2], 0);
    } else {
        launch_expert_ffn(a, h->num_cus, stream);
    }
    if (call >= 0) hipEventRecord(prof_event(h, call, 2), stream);
    launch_combine(a, stream);
    if (call >= 0) hipEventRecord(prof_event(h, call, 3), stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MEGA_MOE_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

int mega_moe_forward(mega_moe_handle* h, int32_t T, const uint8_t* x, const float* x_sf,
                     const int32_t* topk_idx, const float* topk_weights, const uint8_t* w1,
                     const float* w1_sf, const uint8_t* w2, const float* w2_sf, uint16_t* y,
                     void* stream_v) {
    const WeightArgs w{W_FP8_ARGS, w1, w1_sf, nullptr, w2, w2_sf, nullptr};
    return forward_impl(h, T, x, x_sf, topk_idx, topk_weights, w, y, stream_v);
}

int mega_moe_forward_mxfp4(mega_moe_handle* h, int32_t T, const uint8_t* x, const float* x_sf,
                           const int32_t* topk_idx, const float* topk_weights, const uint8_t* w1,
                           const uint8_t* w1_scale, const uint8_t* w2, const uint8_t* w2_scale,
                           uint16_t* y, void* stream_v) {
    const WeightArgs w{W_MXFP4_ARGS, w1, nullptr, w1_scale, w2, nullptr, w2_scale};
    return forward_impl(h, T, x, x_sf, topk_idx, topk_weights, w, y, stream_v);
}

int mega_moe_get_status(mega_moe_handle* h, void* stream_v) {
    if (!h) return fail(MEGA_MOE_ERR_INVALID_ARG, "handle is NULL");
    hipStream_t stream = (hipStream_t)stream_v;
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(MEGA_MOE_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
    uint32_t bits = 0;
    uint32_t* dev_err = &h->base.ctrl->error;
    e = hipMemcpy(&bits, dev_err, sizeof bits, hipMemcpyDeviceToHost);
    if (e == hipSuccess && bits) e = hipMemset(dev_err, 0, sizeof bits);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(MEGA_MOE_ERR_HIP, "status read: %s", hipGetErrorString(e));
    ok();
    return (int)bits;
}

int mega_moe_transform_w1(int32_t num_experts, int32_t hidden, int32_t intermediate,
                          const uint8_t* w1_plain, const float* w1_sf_plain, uint8_t* w1_out,
                          float* w1_sf_out, void* stream_v) {
    if (num_experts < 1 || hidden <= 0 || hidden % 128 || intermediate <= 0 || intermediate % 128)
        return fail(MEGA_MOE_ERR_INVALID_ARG,
                    "need num_experts >= 1 and hidden, intermediate positive multiples of 128");
    if (!w1_plain || !w1_sf_plain || !w1_out || !w1_sf_out)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned(w1_plain, 8) || !aligned(w1_out, 8) || !aligned(w1_sf_plain, 4) ||
        !aligned(w1_sf_out, 4))
        return fail(MEGA_MOE_ERR_INVALID_ARG, "codes must be 8-byte and scales 4-byte aligned");
    const size_t bytes = (size_t)num_experts * 2 * intermediate * hidden;
    const uintptr_t a0 = (uintptr_t)w1_plain, b0 = (uintptr_t)w1_out;
    if (a0 < b0 + bytes && b0 < a0 + bytes)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "w1_plain and w1_out overlap");
    launch_transform_w1(w1_plain, w1_sf_plain, w1_out, w1_sf_out, num_experts, 2 * intermediate,
                        hidden, (hipStream_t)stream_v);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MEGA_MOE_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

int mega_moe_set_recv_stats(mega_moe_handle* h, int32_t* stats) {
    if (!h) return fail(MEGA_MOE_ERR_INVALID_ARG, "handle is NULL");
    if (!aligned(stats, 4)) return fail(MEGA_MOE_ERR_INVALID_ARG, "stats must be 4-byte aligned");
    h->base.recv_stats = stats;
    return ok();
}

int mega_moe_profile_begin(mega_moe_handle* h, int32_t max_calls) {
    if (!h) return fail(MEGA_MOE_ERR_INVALID_ARG, "handle is NULL");
    if (max_calls < 1 || max_calls > 4096)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "max_calls must be in [1, 4096]");
    prof_release(h);
    h->prof_events.resize((size_t)max_calls * 4, nullptr);
    for (auto& ev : h->prof_events) {
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) {
            ev = nullptr;
            prof_release(h);
            return fail(MEGA_MOE_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
        }
    }
    h->prof_max = max_calls;
    h->prof_used = 0;
    return ok();
}

int mega_moe_profile_end(mega_moe_handle* h, float* ms_out, int32_t capacity, int32_t* n_out) {
    if (!h || !n_out || (capacity > 0 && !ms_out))
        return fail(MEGA_MOE_ERR_INVALID_ARG, "NULL argument");
    const int n = h->prof_used < capacity ? h->prof_used : capacity;
    for (int c = 0; c < n; ++c) {
        hipError_t e = hipEventSynchronize(prof_event(h, c, 3));
        for (int k = 0; k < 3 && e == hipSuccess; ++k)
            e = hipEventElapsedTime(&ms_out[c * 3 + k], prof_event(h, c, k), prof_event(h, c, k + 1));
        if (e != hipSuccess) {
            prof_release(h);
            return fail(MEGA_MOE_ERR_HIP, "event timing: %s", hipGetErrorString(e));
        }
    }
    *n_out = n;
    prof_release(h);
    return ok();
}

int mega_moe_get_views(mega_moe_handle* h, mega_moe_views* v) {
    if (!h || !v) return fail(MEGA_MOE_ERR_INVALID_ARG, "NULL argument");
    const MoeArgs& a = h->base;
    v->counts = a.counts;
    v->offsets = a.offsets;
    v->slot_map = a.slot_map;
    v->src = a.src;
    const bool pool = h->cfg.keep_pool != 0;
    v->l1_acts = pool ? a.l1_acts : nullptr;
    v->l1_acts_sf = pool ? a.l1_sf : nullptr;
    v->l1_topk_weights = pool ? a.l1_w : nullptr;
    v->l2_acts = a.l2_acts;
    v->l2_acts_sf = a.l2_sf;
    v->combine_buf = a.comb;
    v->pool_rows_capacity = a.P_cap;
    v->last_num_tokens = h->last_T;
    return ok();
}

// ---------------------------------------------------------------------------
// Allocation-free forward.  Its workspace is the file-scope device array
// `scratch` below: every GPU the library runs on holds its own copy of it
// until the process ends.  Host code never uses the array's name as an
// address (in host code it is only a stand-in for the symbol): the set-up
// of each device asks the runtime for that device's address of it, once,
// with the device current, and every kernel argument is derived from that.
// The control record (queue heads, error bits) sits at its start, the
// per-call layout after it.
// ---------------------------------------------------------------------------
constexpr int64_t NOALLOC_CTRL_BYTES = 256;
static_assert(sizeof(MoeCtrl) <= NOALLOC_CTRL_BYTES, "control record");

int mega_moe_forward_noalloc(const mega_moe_config* cfg, int32_t T, const uint8_t* x,
                             const float* x_sf, const int32_t* topk_idx,
                             const float* topk_weights, const uint8_t* w1, const float* w1_sf,
                             const uint8_t* w2, const float* w2_sf, uint16_t* y,
                             uint32_t* dev_errors, void* stream_v);

}  // extern "C"

static __device__ __align__(256) uint8_t scratch[MEGA_MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;

struct NoallocDevice {
    std::once_flag once;
    int rc = MEGA_MOE_OK;
    std::string err;
    uint8_t* ptr = nullptr;       // this device's address of `scratch`
    int num_cus = 0, n_xcd = 0;
    std::mutex clear_mu;
    bool cleared = false;         // the control record's first clear was issued
};

NoallocDevice g_noalloc[NOALLOC_MAX_DEVICES];

// One-time set-up of device dev (current on the calling thread): the device
// checks of mega_moe_create (without its probe kernel, which would
// synchronise) and the device address of `scratch`.
void noalloc_setup(NoallocDevice& d, int dev) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
        d.rc = fail(MEGA_MOE_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    } else if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        d.rc = fail(MEGA_MOE_ERR_UNSUPPORTED, "device %d is %s, this library is built for gfx950",
                    dev, prop.gcnArchName);
    } else if ((d.rc = xcd_count(dev, prop.multiProcessorCount, &d.n_xcd)) == MEGA_MOE_OK) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            d.rc = fail(MEGA_MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        } else {
            d.ptr = static_cast<uint8_t*>(p);
            d.num_cus = prop.multiProcessorCount;
        }
    }
    if (d.rc) d.err = g_last_error;
}

}  // namespace

extern "C" {

int mega_moe_forward_noalloc(const mega_moe_config* cfg, int32_t T, const uint8_t* x,
                             const float* x_sf, const int32_t* topk_idx,
                             const float* topk_weights, const uint8_t* w1, const float* w1_sf,
                             const uint8_t* w2, const float* w2_sf, uint16_t* y,
                             uint32_t* dev_errors, void* stream_v) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (cfg->keep_pool || cfg->split_l2_cus || cfg->split_l2_xcds)
        return fail(MEGA_MOE_ERR_INVALID_ARG,
                    "the allocation-free forward takes neither keep_pool nor a split");
    if (T < 0 || T > cfg->max_tokens)
        return fail(MEGA_MOE_ERR_INVALID_ARG, "num_tokens %d outside [0, max_tokens=%d]", T,
                    cfg->max_tokens);
    if (T == 0) return ok();
    const WeightArgs w{W_FP8_ARGS, w1, w1_sf, nullptr, w2, w2_sf, nullptr};
    rc = check_tensors(x, x_sf, topk_idx, topk_weights, w, y);
    if (rc) return rc;
    if (dev_errors && !aligned(dev_errors, 4))
        return fail(MEGA_MOE_ERR_INVALID_ARG, "dev_errors must be 4-byte aligned");
    // the layout of this call: the workspace of a handle sized for T tokens
    mega_moe_config c = *cfg;
    c.max_tokens = T;
    const Layout L = make_layout(c);
    const int64_t need = NOALLOC_CTRL_BYTES + L.total;
    if (need > (int64_t)MEGA_MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MEGA_MOE_ERR_INVALID_ARG,
                    "%d tokens need %lld bytes of scratch; the allocation-free forward has %lld "
                    "(use a handle from mega_moe_create for larger batches)", T, (long long)need,
                    (long long)MEGA_MOE_NOALLOC_SCRATCH_BYTES);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MEGA_MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return fail(MEGA_MOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev,
                    NOALLOC_MAX_DEVICES);
    NoallocDevice& d = g_noalloc[dev];
    std::call_once(d.once, noalloc_setup, std::ref(d), dev);
    if (d.rc) return fail(d.rc, "%s", d.err.c_str());
    hipStream_t stream = (hipStream_t)stream_v;
    {
        // the control record starts cleared (device globals are zero-filled
        // when the code object loads; this first clear does not rely on it)
        std::lock_guard<std::mutex> lk(d.clear_mu);
        if (!d.cleared) {
            launch_clear_words(reinterpret_cast<uint32_t*>(d.ptr),
                               (int)(NOALLOC_CTRL_BYTES / 4), stream);
            d.cleared = true;
        }
    }
    MoeArgs a;
    bind_workspace(a, c, L, d.ptr + NOALLOC_CTRL_BYTES, d.n_xcd);
    a.ctrl = reinterpret_cast<MoeCtrl*>(d.ptr);
    a.err_move = 1;
    a.err_out = dev_errors;
    call_args(a, c, T, x, x_sf, topk_idx, topk_weights, w, y);
    launch_dispatch(a, 0, stream);
    launch_expert_ffn(a, d.num_cus, stream);
    launch_combine(a, stream);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(MEGA_MOE_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
