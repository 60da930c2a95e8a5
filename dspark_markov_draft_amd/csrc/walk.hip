// Host side of the dense walk: which kernel runs, how W2 is split over the grid, the launch.
//
// Path: one request multiplies every W2 row by one W1 row (a GEMV), which the lane-per-row
// v_dot4 kernel does at full VALU rate; two or more requests make each step a GEMM that the
// int8 matrix cores (v_mfma_i32_16x16x64_i8, ~12x the MACs per cycle of v_dot4 on gfx950) run
// 16 requests at a time.
//
// Partition: workgroup w owns the contiguous rows [w * rpw, (w + 1) * rpw) (the last one
// fewer); rpw is the smallest multiple of 4 (v_dot4) or 16 (MFMA tiles) that covers V with at
// most one workgroup per compute unit, and at least 256 rows unless V is smaller. Within a
// workgroup the rows go first to VGPRs, then to LDS, and any rest is streamed every step.
#include "walk_common.hpp"

namespace dspark {

constexpr int DOT4_LDS_SETS_MAX = 2;    // row sets in LDS
// LDS besides the W2 rows: W1 high digits, their steps, wave keys, tokens; then the low digits
// (all requests' in the lane-per-row kernel, the one request's in the one-request MFMA kernel)
constexpr int WALK_FIXED_LDS = W1Q_BYTES + MAX_BS * 4 + WALK_WAVES * MAX_BS * 8 + MAX_BS * 4;
constexpr int DOT4_FIXED_LDS = WALK_FIXED_LDS + W1L_BYTES;
constexpr int MFMA1_FIXED_LDS = WALK_FIXED_LDS + RANK + MFMA1_MAX_GROUPS * WAVE * 4;
constexpr int MFMA_REG_TILES = 8;       // 16-row tiles per wave in VGPRs
constexpr int MFMA_TILE_LDS = 4 * WAVE * 16;
// Smallest batch run on the MFMA kernel: below it the lane-per-row kernel is faster (measured at
// V = 151936, 7 steps: 48 vs 63 us greedy at bs 1, 60 vs 64 at bs 2, 85 vs 67 at bs 4; sampling
// moves the crossover up by one request, its finish costing more per MFMA tile).
constexpr int MFMA_MIN_BS_GREEDY = 3;
constexpr int MFMA_MIN_BS_SAMPLE = 4;
// Waves per workgroup of the MFMA kernel with static LDS (4 or 8; the test hook
// DSPARK_DEBUG_MFMA_WAVES forces either); the kernel with dynamic LDS has 4.
constexpr int MFMA_STATIC_WAVES = 8;

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

static int plan_path(const DeviceInfo& dev, int cap, int64_t bs, int64_t V, int path, int sample,
                     dspark_walk_plan* plan) {
    int waves = WALK_WAVES;
    const int64_t quantum = path == DSPARK_PATH_MFMA ? 16 : 4;   // (MFMA1 handles partial tiles)
    int64_t rpw = (V + cap - 1) / cap;
    if (rpw < WALK_THREADS) rpw = V < WALK_THREADS ? V : WALK_THREADS;
    rpw = round_up(rpw, quantum);
    const int64_t nwg = (V + rpw - 1) / rpw;

    int64_t reg_rows, lds_rows, units, reg_units, lds_units, lds_bytes;
    int64_t stage_bufs = 0, stage_stride = 0;
    if (path == DSPARK_PATH_MFMA1) {
        // one request: every row on chip as 16-row tiles, MFMA1_TILES per wave in registers,
        // up to MFMA1_LDS_TILES more in LDS
        if (rpw > MFMA1_MAX_ROWS) return DSPARK_ERR_UNSUPPORTED;   // the caller falls back
        units = ((rpw + 15) / 16 + WALK_WAVES - 1) / WALK_WAVES;   // tiles per wave
        reg_units = units < MFMA1_TILES ? units : MFMA1_TILES;
        lds_units = units - reg_units;
        reg_rows = rpw < reg_units * WALK_WAVES * 16 ? rpw : reg_units * WALK_WAVES * 16;
        lds_rows = rpw - reg_rows;
        // (the variant with LDS slots always has MFMA1_LDS_TILES of them)
        lds_bytes = (lds_units ? MFMA1_LDS_TILES : 0) * WALK_WAVES * MFMA_TILE_LDS + MFMA1_FIXED_LDS;
    } else if (path == DSPARK_PATH_DOT4) {
        units = (rpw + WALK_THREADS - 1) / WALK_THREADS;            // row sets
        reg_units = units < DOT4_REG_SETS ? units : DOT4_REG_SETS;
        lds_units = units - reg_units;
        if (lds_units > DOT4_LDS_SETS_MAX) lds_units = DOT4_LDS_SETS_MAX;
        const int64_t room = ((int64_t)dev.max_lds - DOT4_FIXED_LDS) / (WALK_THREADS * RANK);
        if (lds_units > room) lds_units = room > 0 ? room : 0;
        reg_rows = rpw < reg_units * WALK_THREADS ? rpw : reg_units * WALK_THREADS;
        lds_rows = rpw - reg_rows;
        if (lds_rows > lds_units * WALK_THREADS) lds_rows = lds_units * WALK_THREADS;
        lds_bytes = lds_units * WALK_THREADS * RANK + DOT4_FIXED_LDS;
    } else {
        // staging buffers for the base logits of a 16-request tile come first (rows padded to an
        // odd number of 16-byte units); two when there is more than one request tile
        int64_t u16 = rpw / 4;
        if (u16 % 2 == 0) u16 += 1;
        stage_stride = u16 * 4;
        int64_t buf_bytes = 16 * stage_stride * 4;
        const int64_t fixed = mfma_fixed_lds_bytes((int)rpw);
        const int64_t want = bs > 16 ? 2 : 1;
        const bool stat = rpw <= MFMA_STATIC_ROWS && stage_stride <= MFMA_STATIC_STRIDE;
        const int64_t dyn_max = (int64_t)dev.max_lds - MFMA_DYN_STATIC_RESERVE;   // without STAT
        const int forced = debug_knobs().mfma_waves;
        if (stat) waves = forced ? forced : MFMA_STATIC_WAVES;
        const int64_t tiles = rpw / 16;
        units = (tiles + waves - 1) / waves;                        // tile slots per wave
        const int slots = mfma_static_slots((int)units, waves);     // of the static build
        if (stat) {
            // all LDS is static and of fixed size (both staging buffers exist for any batch)
            stage_bufs = want;
            if (mfma_static_lds_bytes(sample, slots, waves) > (int64_t)dev.max_lds)
                return DSPARK_ERR_UNSUPPORTED;
        } else {
            stage_bufs = (dyn_max - fixed) / buf_bytes;
            if (stage_bufs > want) stage_bufs = want;
            if (stage_bufs < 1) return DSPARK_ERR_UNSUPPORTED;    // the caller falls back
        }
        const int64_t stage_lds = stage_bufs * buf_bytes;
        const int64_t reg_tiles = stat ? slots - mfma_static_lds_slots(slots, waves) : MFMA_REG_TILES;
        reg_units = units < reg_tiles ? units : reg_tiles;
        int64_t room = stat ? mfma_static_lds_slots(slots, waves)
                            : (dyn_max - fixed - stage_lds) / (WALK_WAVES * MFMA_TILE_LDS);
        if (room < 0) room = 0;
        lds_units = units - reg_units;
        if (lds_units > room) lds_units = room;
        reg_rows = rpw < reg_units * waves * 16 ? rpw : reg_units * waves * 16;
        lds_rows = rpw - reg_rows;
        if (lds_rows > lds_units * waves * 16) lds_rows = lds_units * waves * 16;
        lds_bytes = stat ? mfma_static_lds_bytes(sample, slots, waves)
                         : lds_units * WALK_WAVES * MFMA_TILE_LDS + fixed + stage_lds;
        if (!stat && lds_bytes > dyn_max) return DSPARK_ERR_UNSUPPORTED;
    }
    if (lds_bytes < LDS_MIN_BYTES) lds_bytes = LDS_MIN_BYTES;
    if ((size_t)lds_bytes > dev.max_lds) return DSPARK_ERR_UNSUPPORTED;

    // whole-grid byte counts: rows are owned contiguously, the last workgroup may own fewer
    int64_t res = 0, str = 0;
    for (int64_t w = 0; w < nwg; ++w) {
        const int64_t n = (w + 1) * rpw <= V ? rpw : V - w * rpw;
        const int64_t on_chip = n < reg_rows + lds_rows ? n : reg_rows + lds_rows;
        res += on_chip;
        str += n - on_chip;
    }
    plan->device_cus = dev.cus;
    plan->num_workgroups = (int32_t)nwg;
    plan->rows_per_workgroup = (int32_t)rpw;
    plan->rows_in_registers = (int32_t)reg_rows;
    plan->rows_in_lds = (int32_t)lds_rows;
    plan->rows_streamed = (int32_t)(rpw - reg_rows - lds_rows);
    plan->resident_bytes = res * RANK;
    plan->streamed_bytes = str * RANK;
    plan->lds_bytes = (int32_t)lds_bytes;
    plan->path = path;
    plan->reg_units = (int32_t)reg_units;
    plan->lds_units = (int32_t)lds_units;
    plan->total_units = (int32_t)units;
    plan->stage_bufs = (int32_t)stage_bufs;
    plan->stage_stride = (int32_t)stage_stride;
    plan->waves_per_workgroup = waves;
    return DSPARK_OK;
}

// The MFMA kernel runs from MFMA_MIN_BS_* requests when V % 4 == 0 (and, at launch, the rows it
// moves as vectors are 16-byte aligned) and its staging buffer fits in LDS; otherwise, or when
// forced by the test hook, the v_dot4 kernel runs.
int plan_walk(const DeviceInfo& dev, int64_t bs, int64_t T, int64_t V, int sample,
              dspark_walk_plan* plan) {
    (void)T;
    int cap = dev.cus < MAX_WORKGROUPS ? dev.cus : MAX_WORKGROUPS;
    const DebugKnobs& dbg = debug_knobs();
    if (dbg.max_workgroups > 0 && dbg.max_workgroups < cap) cap = dbg.max_workgroups;
    if (cap < 1) return DSPARK_ERR_NO_DEVICE;
    const int min_bs = sample ? MFMA_MIN_BS_SAMPLE : MFMA_MIN_BS_GREEDY;
    int path = (bs >= min_bs && V % 4 == 0) ? DSPARK_PATH_MFMA
               : bs == 1                      ? DSPARK_PATH_MFMA1
                                              : DSPARK_PATH_DOT4;
    if (dbg.force_path == DSPARK_PATH_DOT4) path = DSPARK_PATH_DOT4;
    if (dbg.force_path == DSPARK_PATH_MFMA && V % 4 == 0) path = DSPARK_PATH_MFMA;
    if (dbg.force_path == DSPARK_PATH_MFMA1 && bs == 1) path = DSPARK_PATH_MFMA1;
    if (path != DSPARK_PATH_DOT4 && plan_path(dev, cap, bs, V, path, sample, plan) == DSPARK_OK)
        return DSPARK_OK;
    return plan_path(dev, cap, bs, V, DSPARK_PATH_DOT4, sample, plan);
}

// The kernels' waits need all their workgroups resident at once. The grid never exceeds the
// compute units, and each workgroup asks for more than half of a CU's LDS, so each CU holds at
// most one; with the device otherwise idle they are all resident. If they are not (other work
// holds CUs), the waits run into their time bound and the call reports DSPARK_ERR_TIMEOUT
// instead of hanging. A cooperative launch would guarantee residency but costs ~20 us per
// launch on this stack, an order of magnitude above a plain launch.
int launch_dense_walk(const WalkLaunch& a, const dspark_walk_plan& plan_in, hipStream_t stream) {
    dspark_walk_plan plan = plan_in;
    const bool vec_ok = (a.V % 4 == 0) && ((uintptr_t)a.base % 16 == 0) &&
                        ((uintptr_t)a.draft_logits % 8 == 0) && ((uintptr_t)a.out_logits % 16 == 0);
    if (plan.path == DSPARK_PATH_MFMA && !vec_ok) {
        DeviceInfo dev;
        if (current_device_info(&dev) != DSPARK_OK) return DSPARK_ERR_NO_DEVICE;
        int cap = dev.cus < MAX_WORKGROUPS ? dev.cus : MAX_WORKGROUPS;
        const int dbg_cap = debug_knobs().max_workgroups;
        if (dbg_cap > 0 && dbg_cap < cap) cap = dbg_cap;
        const int st = plan_path(dev, cap, a.bs, a.V, DSPARK_PATH_DOT4, a.sample, &plan);
        if (st != DSPARK_OK) return st;
    }
    WalkParams p;
    p.q = a.q;
    p.scale = a.scale;
    p.w1 = a.w1;
    p.base = a.base;
    p.start = a.start;
    p.tokens = a.tokens;
    p.out_logits = a.out_logits;
    p.draft_logits = a.draft_logits;
    p.seeds = a.seeds;
    p.positions = a.positions;
    p.temps = a.temps;
    char* ws = static_cast<char*>(a.workspace);
    p.result = reinterpret_cast<uint64_t*>(ws + WS_RESULT);
    p.slots = reinterpret_cast<uint64_t*>(ws + WS_SLOTS);
    p.err = a.error_word ? a.error_word : reinterpret_cast<uint32_t*>(ws + WS_ERR);
    p.done = reinterpret_cast<uint64_t*>(ws + WS_ICDF_DONE);
    p.never = reinterpret_cast<const uint32_t*>(ws + WS_ERR + 4);
    p.bs = a.bs;
    p.T = a.T;
    p.V = a.V;
    p.rows_per_wg = plan.rows_per_workgroup;
    p.reg_units = plan.reg_units;
    p.lds_units = plan.lds_units;
    p.total_units = plan.total_units;
    p.stride = slot_stride(a.bs);
    p.stage_bufs = plan.stage_bufs;
    p.stage_stride = plan.stage_stride;
    p.vec_ok = vec_ok ? 1 : 0;
    p.w1_row_bytes = RANK * (a.w1_dtype == DSPARK_F32 ? 4 : 2);
    const DebugKnobs& dbg = debug_knobs();
    p.spin_ticks = dbg.spin_ticks ? dbg.spin_ticks : DEFAULT_SPIN_TICKS;
    p.wait_unset = dbg.wait_unset ? 1 : 0;
    p.stamps = reinterpret_cast<uint64_t*>(dbg.stamps);
    const bool timed = p.stamps != nullptr && a.w1_dtype == DSPARK_BF16 && a.sample != 2;

    const int w1t = a.w1_dtype == DSPARK_F32 ? DT_F32 : a.w1_dtype == DSPARK_BF16 ? DT_BF16 : DT_F16;
    // the MFMA kernel for small slices keeps all its LDS in static arrays (no dynamic LDS)
    const bool static_stage = plan.path == DSPARK_PATH_MFMA &&
                              plan.rows_per_workgroup <= MFMA_STATIC_ROWS &&
                              plan.stage_stride <= MFMA_STATIC_STRIDE;
    const int dyn_lds = static_stage ? 0 : plan.lds_bytes;
    const void* fn = plan.path == DSPARK_PATH_MFMA
                         ? mfma_walk_kernel(a.sample, w1t, timed, static_stage,
                                            a.out_logits != nullptr,
                                            mfma_static_slots(plan.total_units, plan.waves_per_workgroup),
                                            plan.waves_per_workgroup)
                     : plan.path == DSPARK_PATH_MFMA1
                         ? mfma1_walk_kernel(a.sample, w1t, timed, plan.lds_units > 0,
                                             mfma1_reg_slots(plan.total_units))
                                                       : dot4_walk_kernel(a.sample, w1t, timed);
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, dyn_lds) !=
        hipSuccess) {
        (void)hipGetLastError();
    }
    void* args[] = {&p};
    const int threads = plan.path == DSPARK_PATH_MFMA ? plan.waves_per_workgroup * WAVE : WALK_THREADS;
    const hipError_t e = launch_walk_kernel(fn, dim3(plan.num_workgroups), dim3(threads),
                                            args, (size_t)dyn_lds, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return DSPARK_ERR_LAUNCH;
    }
    return DSPARK_OK;
}

}  // namespace dspark
