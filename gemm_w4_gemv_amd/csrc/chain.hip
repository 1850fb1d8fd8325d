// Persistent decode-chain kernel: a whole sequence of dependent INT4 GEMVs in
// one launch.
//
// "Lab 5: Gemma4 端到端推理优化", sections "CUDA Graph" and "性能分析": once
// the GEMVs were fused, the decode step's remaining cost was fixed per-launch
// overhead, so the step is captured and replayed as one unit.  On MI355X a
// graph node still costs about 1.8 us and every dependent kernel boundary
// drains and refills HBM (about 4 us of ramp and tail per GEMV), which for a
// 336-GEMV step is as much time as its 5.7 GB of weights take to stream.  This
// kernel removes the boundaries; a persistent kernel fusing several GEMMs into
// one launch is the remedy named in "在 Triton 中利用 Cutlass 内核命名解锁 FP8
// 张量核心加速" (its last paragraph).
//
// The chain is a list of stages.  GEMVs of one stage are independent (q, k, v;
// gate, up); a GEMV of stage s may read, as its x, the output of a GEMV of an
// earlier stage.  One 768-thread workgroup runs per compute unit, its 12
// waves (three per SIMD) in two roles:
//
//  * kChainComputeWaves compute waves.  The tiles of each stage are split
//    evenly over all compute waves of the GPU.  A tile is kChainTileRows
//    slot-rows of 2 chunks (16 bytes of codes) per lane; x comes from LDS.
//    A wave keeps three tiles in flight in three register sets used in turn:
//    while one is computed the next two load, and the set just computed is
//    refilled with the tile three ahead (a dummy load of an empty buffer
//    range past the wave's last tile, so every step issues the same loads
//    and the compiler's wait counts stay exact).  A wave publishes, in its own LDS
//    word, how many stages it has finished; it never waits for its own stores.
//  * Staging waves (the rest).  Stage t's x vectors go into LDS buffer t & 1
//    in the dot2 pair layout once every compute wave of the workgroup is past
//    stage t - 2; the staging waves split the stage's 64-chunk slots.  An
//    input from outside the chain is loaded as soon as the buffer is free.
//    An input that is an earlier GEMV's output is read from that GEMV's
//    copy in the workspace (bf16, written by the producer with
//    device-coherent stores): the staging waves poll it with device-coherent
//    loads until none of its values is the empty mark (a NaN pattern),
//    starting once their own workgroup has finished the producing stage.
//
// So a GEMV waits for exactly the outputs it reads, and nothing else
// synchronises workgroups: there is no grid-wide barrier.  Each workgroup
// counts its launches in its own workspace line.  The copies come in two
// halves: a launch writes and polls the half of its count's parity, and its
// staging waves first mark the other half empty for the next launch (launches
// of one chain run one after another, so nothing reads that half meanwhile).
// A copy holds two bytes per value, half of what a value tagged with its
// writer would take: every workgroup polls every input it stages, so the
// polls' bytes are on the critical path of each boundary.
// Every wait is bounded: past the spin limit
// the waiter records an error in the workspace and goes on (a staging wave
// stops staging), so the launch always ends.
#include "chain.hpp"
#include "gemv_common.hpp"

namespace w4 {

#ifdef W4_CHAIN_TIMELINE
// Timeline build only (chain_timeline.py): per workgroup and stage, four
// s_memrealtime stamps (100 MHz) of the last launch: [0] its staging starts
// (first staging wave), [1] its x is staged (last staging wave), [2] its
// first tile's math starts (first compute wave), [3] its last tile's loads
// for later stages are issued (last compute wave).  Workgroups and stages
// past the bounds below are not recorded.
constexpr int kTimelineStages = 512;
constexpr int kTimelineWorkers = 256;
__device__ unsigned g_chain_timeline[kTimelineWorkers * kTimelineStages * 4];
#endif

namespace {

// Tile shape.  A tile is kSlotRows slot-rows x 2 chunks per lane.  A row of
// C <= 128 chunks fills one slot-row; a longer row is cut into sp = 2 or 4
// segments of 128 chunks on consecutive slot-rows, whose partial sums are
// added after the cross-lane reduction.
// Slot-row q holds segment (q % sp) of row (q / sp); lane l's chunks in it
// are 128 (q % sp) + l and + l + 64, in groups 32 (q % sp) + (l + 64 i) / 4.
constexpr int kSlotRows = kChainTileRows;
constexpr int kSlotLanes = kWave / kSlotRows;  // lanes per slot-row after the row reduction

struct TileRegs {
    u32x4_t w[2 * kSlotRows];  // slot (q, i) in w[2 q + i]
    // Per slot-row, one 16-bit value per lane: lane l < 32 holds the scale of
    // group l of the slot-row's segment, lane l >= 32 the zero of group l - 32.
    // Each lane's own pair is gathered from these at use (one VGPR per
    // slot-row; loading each lane's four values would take three more, past
    // the register budget of four waves per SIMD).
    uint16_t sz[kSlotRows];
};

// A compute wave's position: tile t of stage s, i.e. rows [row, row + nrows)
// of GEMV g; end = end of the wave's tile range in the stage.
struct Work {
    int s, t, end, g, row, nrows;
};

struct Shared {
    // Stages each compute wave has finished with (its LDS x no longer
    // needed).  One word per wave, not a shared count: a wave with no tiles
    // in the next stages reports several at once, and a sum would then run
    // ahead of waves still working on an earlier stage.
    unsigned progress[kChainComputeWaves];
    // Stages each staging wave has staged; per wave for the same reason.
    unsigned staged[kChainStagers];
    unsigned abort;
    unsigned timed_out;  // a compute wave stopped waiting for its x (recorded at the end)
    unsigned base;       // launches this workgroup has run before this one
    uint32_t mirror_off;  // byte offset of this launch's half of the copies: (base & 1) * mirror_half_bytes
#ifdef W4_CHAIN_TIMELINE
    unsigned timeline[kTimelineStages * 4];
#endif
};

// Timeline stamp (timeline build only; called by one lane): the earliest or
// the latest time event e of stage t was reached in this workgroup.
__device__ __forceinline__ void timeline_mark(Shared& sh, int t, int e, bool earliest) {
#ifdef W4_CHAIN_TIMELINE
    if (t < kTimelineStages) {
        const unsigned now = (unsigned)__builtin_amdgcn_s_memrealtime();
        unsigned* p = &sh.timeline[t * 4 + e];
        if (earliest) __hip_atomic_fetch_min(p, now, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        else __hip_atomic_fetch_max(p, now, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
#else
    (void)sh, (void)t, (void)e, (void)earliest;
#endif
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Neither BF16 half of a polled word is the empty mark.
__device__ __forceinline__ unsigned filled(uint32_t w) {
    return (unsigned)((w & 0xFFFFu) != kChainMirrorEmpty) & (unsigned)((w >> 16) != kChainMirrorEmpty);
}

// s_waitcnt immediate that waits for vmcnt <= n only (expcnt and lgkmcnt at
// their maxima): vmcnt bits 3:0 and 15:14.
constexpr unsigned vmcnt_imm(unsigned n) { return (n & 15u) | 0x70u | 0xF00u | ((n >> 4) << 14); }
static_assert(vmcnt_imm(0) == 0xF70u && vmcnt_imm(12) == 0xF7Cu && vmcnt_imm(24) == 0x4F78u, "vmcnt encoding");
__device__ __forceinline__ int seg_shift(int sp) { return sp == 1 ? 0 : (sp == 2 ? 1 : 2); }

__device__ __forceinline__ unsigned lds_load(const unsigned* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void set_error(const ChainLaunch& L, Shared& sh, unsigned bit) {
    __hip_atomic_fetch_or(L.err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&sh.abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Place ``w`` at tile w.t of stage w.s.  Every field is wave-uniform;
// readfirstlane tells the compiler so, keeping the work state and the buffer
// descriptors built from it in SGPRs.  The GEMV holding the tile is found by
// a binary search over the stage's tile0 table (ascending) when ``from`` is
// -1, else by a forward scan from GEMV ``from``, which holds an earlier tile
// of the same stage (a wave's tiles of a stage are consecutive).
__device__ __forceinline__ void place(const ChainLaunch& L, Work& w, int from) {
    const ChainStage st = L.stages[w.s];
    int g;
    if (from < 0) {
        int lo = st.gemv0, hi = st.gemv0 + st.ngemv - 1;  // the answer lies in [lo, hi]
        while (lo < hi) {
            const int mid = uniform((lo + hi + 1) >> 1);
            if (w.t >= L.gemvs[mid].tile0) lo = mid;
            else hi = mid - 1;
        }
        g = lo;
    } else {
        g = from;
        while (g + 1 < st.gemv0 + st.ngemv && w.t >= L.gemvs[g + 1].tile0) g = uniform(g + 1);
    }
    g = uniform(g);
    const ChainGemv& G = L.gemvs[g];
    const int rpt = kSlotRows / G.sp;
    w.g = g;
    w.row = uniform((w.t - G.tile0) * rpt);
    w.nrows = uniform(min(rpt, G.N - w.row));
}

// First work at or after stage s for compute wave v of W (s == num_stages:
// none).  The tiles of a stage are split evenly over the W compute waves.
__device__ __forceinline__ Work first_from(const ChainLaunch& L, int s, int v, int W) {
    Work w{};
    for (; s < L.num_stages; ++s) {
        const int tiles = L.stages[s].tiles;
        const int a = uniform((int)(((long long)v * tiles) / W));
        const int b = uniform((int)(((long long)(v + 1) * tiles) / W));
        if (a < b) {
            w.s = uniform(s);
            w.t = a;
            w.end = b;
            place(L, w, -1);
            return w;
        }
    }
    w.s = uniform(L.num_stages);
    return w;
}

__device__ __forceinline__ Work advance(const ChainLaunch& L, Work w, int v, int W) {
    w.t = uniform(w.t + 1);
    if (w.t < w.end) {
        place(L, w, w.g);
        return w;
    }
    return first_from(L, w.s + 1, v, W);
}

// Issue the loads of one tile: 8 weight loads and 4 scale/zero loads (no wait).  A dummy issue (past a
// wave's last tile) repeats w's scale/zero loads and gives its weight loads
// an empty buffer range, which returns zeros without touching memory: the
// same loads are issued on every path, so the compiler's wait counts for the
// first tile stay exact.
__device__ __forceinline__ void issue(const ChainGemv& G, const Work& w, bool dummy, int lane, TileRegs& R) {
    const int C = G.C, N = G.N, Gr = C >> 2, sp = G.sp, sh = seg_shift(sp);
    const uint32_t row_bytes = (uint32_t)C * 16u;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(G.qw, dummy ? 0u : (uint32_t)N * row_bytes);
    // Issue order = use order (scales and zeros, then chunk column 0 of every
    // slot-row, then column 1), so the math can start on the first arrivals.
    // A global (not flat) pointer for the scales and zeros: flat loads would
    // also count in lgkmcnt and make every LDS wait wait for the prefetches.
    typedef __attribute__((address_space(1))) const uint16_t g_u16;
    g_u16* sz = (g_u16*)(lane < 32 ? G.s : G.z);
#pragma unroll
    for (int q = 0; q < kSlotRows; ++q) {
        const int row = w.row + min(q >> sh, w.nrows - 1);
        const int grp = min(32 * (q & (sp - 1)) + (lane & 31), Gr - 1);
        R.sz[q] = sz[(size_t)row * Gr + grp];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int q = 0; q < kSlotRows; ++q) {
            const uint32_t row = (uint32_t)(w.row + min(q >> sh, w.nrows - 1));
            const uint32_t c = (uint32_t)min(128 * (q & (sp - 1)) + lane + kWave * i, C - 1);
            R.w[2 * q + i] = buf_load_b128<kAuxNontemporal>(rw, c * 16u, row * row_bytes);
        }
    }
}

// x of one chunk from the LDS staging buffer: 16 words of dot2 pairs and
// the chunk sum (chunks past the row end are staged as zeros).
__device__ __forceinline__ float lds_x_chunk(const unsigned char* xg, int Cp, int c, uint32_t xp[16]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xg + ((size_t)p * Cp + c) * 16);
        xp[4 * p + 0] = v.x;
        xp[4 * p + 1] = v.y;
        xp[4 * p + 2] = v.z;
        xp[4 * p + 3] = v.w;
    }
    return *reinterpret_cast<const float*>(xg + (size_t)64 * Cp + (size_t)c * 4);
}

// One slot: chunk (q, i) of the tile.  Its group within the segment is
// (l + 64 i) / 4; scale and zero come from the lanes that loaded them (a
// gather, lane l reading lane l / 4 + 16 i, through ds_bpermute).
__device__ __forceinline__ float slot(const TileRegs& R, int q, int i, int lane, const uint32_t xp[16], float sx,
                                      uint32_t bias, float acc) {
    const int gs = (lane + kWave * i) >> 2;  // group within the segment, 0..31
    const uint16_t sb = (uint16_t)__shfl((int)R.sz[q], gs, kWave);
    const uint16_t zbits = (uint16_t)__shfl((int)R.sz[q], 32 + gs, kWave);
    const float d = chunk_dot(R.w[2 * q + i], xp, bias);
    const float zb = f16_to_f32(zbits) + 128.f;
    return __builtin_fmaf(f16_to_f32(sb), __builtin_fmaf(-zb, sx, d), acc);
}

// Compute one tile and store its rows.  ``xg`` is the GEMV's staged x in LDS.
// With a single segment every row of the tile uses the lane's same two x
// chunks, read once per tile.
__device__ __forceinline__ void compute(const ChainGemv& G, const Work& w, int lane, const TileRegs& R,
                                        const unsigned char* xg, uint32_t mirror_off, uint32_t mirror_half_bytes) {
    const int sp = G.sp, Cp = chain_x_chunks(G.C);
    const uint32_t bias = vgpr_const(kInt4BiasPair);
    float acc[kSlotRows];
    // Slot-row q reads segment q mod sp of its row.  Chunk column i of every
    // slot-row first: with one segment the x chunk read for q = 0 serves all
    // four rows, and only one chunk of x is held at a time.
#pragma unroll
    for (int q = 0; q < kSlotRows; ++q) acc[q] = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint32_t xp[16];
        float sx = 0.f;
#pragma unroll
        for (int q = 0; q < kSlotRows; ++q) {
            if (q == 0 || sp > 1) sx = lds_x_chunk(xg, Cp, 128 * (q & (sp - 1)) + lane + kWave * i, xp);
            acc[q] = slot(R, q, i, lane, xp, sx, bias, acc[q]);
            // One slot's x at a time: hoisted LDS reads would need more VGPRs
            // than the two tile register sets leave.
            asm volatile("" : "+v"(acc[q])::"memory");
        }
    }
    float total = reduce_rows<kSlotRows>(acc, lane);  // lane L: slot-row L / kSlotLanes
    // A row's segments sit on consecutive slot-rows: lanes kSlotLanes (and
    // 2 kSlotLanes) apart.
    static_assert(kSlotLanes == 16, "segment sums cross lane bits 4 and 5");
    if (sp >= 2) total = pair_sum<16>(total);
    if (sp == 4) total = pair_sum<32>(total);
    const int j = (lane / kSlotLanes) >> seg_shift(sp);  // row of the tile this lane's total belongs to
    if ((lane & (kSlotLanes * sp - 1)) == 0 && j < w.nrows) {
        const uint16_t v = f32_to_bf16(total);
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(G.y, (uint32_t)G.N * 2u);
        __builtin_amdgcn_raw_buffer_store_b16(v, ry, (int)((w.row + j) * 2), 0, 0);
        if (G.ym) {  // the copy a later GEMV polls for, in this launch's half: one device-coherent store
            // The empty mark is a NaN; an output with exactly its bits is stored as another NaN.
            const uint16_t m = v == kChainMirrorEmpty ? kChainMirrorNaN : v;
            const __amdgpu_buffer_rsrc_t rm = make_rsrc(G.ym, mirror_half_bytes + (uint32_t)G.N * 2u);
            __builtin_amdgcn_raw_buffer_store_b16(m, rm, (int)(mirror_off + (uint32_t)(w.row + j) * 2u), 0,
                                                  kAuxDeviceCoherent);
        }
    }
}

// --------------------------------------------------------------- staging waves

// Slot ``k`` of a stage's x staging: chunks [64 m, 64 m + 64) of GEMV g
// (slots cover each GEMV's padded chunk count).
__device__ __forceinline__ bool stage_slot(const ChainLaunch& L, const ChainStage& st, int k, int& g, int& m) {
    for (int gi = 0; gi < st.ngemv; ++gi) {
        const int n = L.gemvs[st.gemv0 + gi].x_slots;
        if (k < n) {
            g = uniform(st.gemv0 + gi);
            m = uniform(k);
            return true;
        }
        k -= n;
    }
    return false;
}

__device__ __forceinline__ int stage_slots(const ChainLaunch& L, const ChainStage& st) {
    int n = 0;
    for (int gi = 0; gi < st.ngemv; ++gi) n += L.gemvs[st.gemv0 + gi].x_slots;
    return n;
}

// Staging of a stage's x into an LDS buffer: bf16 pairs in the dot2 order
// (word p of chunk c at 16 (p Cp + c)), then the chunk sums; padding chunks
// are zeros.  The staging waves split the stage's slots (slot k goes to
// staging wave k mod kChainStagers), so a stage's x arrives in one round trip.
__device__ __forceinline__ void stage_load(const ChainLaunch& L, int g, int m, int lane, u32x4_t raw[4]) {
    const ChainGemv& G = L.gemvs[g];
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(G.x, (uint32_t)G.C * 64u);
    const uint32_t c = (uint32_t)min(m * kWave + lane, G.C - 1);
#pragma unroll
    for (int p = 0; p < 4; ++p) raw[p] = buf_load_b128<0>(rx, c * 64u + 16u * p, 0);
}

// All 32 values of a polled 64-byte chunk are written (none is the empty mark).
__device__ __forceinline__ bool chunk_filled(const u32x4_t raw[4]) {
    unsigned ok = 1u;
#pragma unroll
    for (int p = 0; p < 4; ++p) ok &= filled(raw[p].x) & filled(raw[p].y) & filled(raw[p].z) & filled(raw[p].w);
    return ok != 0u;
}

// x of chunk m * 64 + lane of GEMV g (and, with ``two``, of chunk m1 * 64 +
// lane of GEMV g1) from the producers' copies in this launch's half: poll
// both (device-coherent loads, bounded; a lane reloads only what is not yet
// complete) until none of their values is the empty mark.  False on
// time-out.
__device__ __forceinline__ bool stage_poll(const ChainLaunch& L, Shared& sh, int g, int m, bool two, int g1, int m1,
                                           int lane, u32x4_t raw[4], u32x4_t raw1[4]) {
    const uint32_t off = sh.mirror_off;
    const ChainGemv& A = L.gemvs[g];
    const ChainGemv& B = L.gemvs[g1];
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A.xm, off + (uint32_t)A.C * 64u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B.xm, off + (uint32_t)B.C * 64u);
    const int ca = m * kWave + lane, cb = m1 * kWave + lane;
    bool da = ca >= A.C;  // padding chunks are staged as zeros
    bool db = !two || cb >= B.C;
    unsigned n = 0;
    for (;;) {
        if (!da) {
#pragma unroll
            for (int p = 0; p < 4; ++p) raw[p] = buf_load_b128_coherent(ra, off + (uint32_t)ca * 64u + 16u * p, 0);
        }
        if (!db) {
#pragma unroll
            for (int p = 0; p < 4; ++p) raw1[p] = buf_load_b128_coherent(rb, off + (uint32_t)cb * 64u + 16u * p, 0);
        }
        if (!da) da = chunk_filled(raw);
        if (!db) db = chunk_filled(raw1);
        if (__builtin_amdgcn_ballot_w64(!(da & db)) == 0) break;
        if (lds_load(&sh.abort) || ++n > L.spin_limit) return false;
        // A short pause: a round trip takes about a microsecond, and longer
        // pauses (8) measured 2 % slower on the decode step.
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

__device__ __forceinline__ void stage_write(const ChainLaunch& L, int g, int m, int lane, const u32x4_t raw[4],
                                            unsigned char* xb) {
    const ChainGemv& G = L.gemvs[g];
    const int C = G.C, Cp = chain_x_chunks(C), c = m * kWave + lane;
    unsigned char* xg = xb + G.x_lds;
    uint32_t xp[16];
    float sum = 0.f;
    if (c < C) {
        sum = x_chunk_pairs(raw, xp);
    } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) xp[k] = 0u;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p)
        *reinterpret_cast<u32x4_t*>(xg + ((size_t)p * Cp + c) * 16) =
            u32x4_t{xp[4 * p], xp[4 * p + 1], xp[4 * p + 2], xp[4 * p + 3]};
    *reinterpret_cast<float*>(xg + (size_t)64 * Cp + (size_t)c * 4) = sum;
}

// This staging wave's share of stage s: slots sid, sid + kChainStagers, ...,
// two at a time (inputs from earlier GEMVs polled together).  False if a
// poll timed out.
__device__ bool stage_share(const ChainLaunch& L, Shared& sh, int s, unsigned char* xb, int lane, int sid) {
    const ChainStage st = L.stages[s];
    const int n = stage_slots(L, st);
    for (int k = sid; k < n;) {
        int g0, m0, g1 = 0, m1 = 0;
        stage_slot(L, st, k, g0, m0);
        u32x4_t r0[4], r1[4];
        if (L.gemvs[g0].x_internal) {
            const bool two = stage_slot(L, st, k + kChainStagers, g1, m1) && L.gemvs[g1].x_internal;
            if (!stage_poll(L, sh, g0, m0, two, two ? g1 : g0, two ? m1 : m0, lane, r0, r1)) return false;
            stage_write(L, g0, m0, lane, r0, xb);
            if (two) stage_write(L, g1, m1, lane, r1, xb);
            k += two ? 2 * kChainStagers : kChainStagers;
            continue;
        }
        const bool two = stage_slot(L, st, k + kChainStagers, g1, m1) && !L.gemvs[g1].x_internal;
        stage_load(L, g0, m0, lane, r0);
        if (two) stage_load(L, g1, m1, lane, r1);
        stage_write(L, g0, m0, lane, r0, xb);
        if (two) stage_write(L, g1, m1, lane, r1, xb);
        k += two ? 2 * kChainStagers : kChainStagers;
    }
    return true;
}

// Bounded LDS wait: true once ``ready()``; false on abort or time-out.
template <class F>
__device__ __forceinline__ bool lds_wait(const ChainLaunch& L, Shared& sh, F ready) {
    unsigned n = 0;
    bool ok = ready(), ab = lds_load(&sh.abort) != 0u;
    while (!ok & !ab & (n <= L.spin_limit)) {
        __builtin_amdgcn_s_sleep(1);
        ++n;
        ok = ready();
        ab = lds_load(&sh.abort) != 0u;
    }
    return ok && !ab;
}

// Staging wave sid (0 .. kChainStagers - 1).  Stage t goes into LDS buffer
// t & 1, which is free once every compute wave of the workgroup has finished
// stage t - 2; the staging waves split its 64-chunk slots.  An input from
// outside the chain is loaded as soon as the buffer is free (while earlier
// stages still run); an input that is an earlier GEMV's output is polled
// from that GEMV's copy until none of its values is the empty mark, so a
// stage waits for exactly the outputs it reads and for nothing else.
// Polling starts once this workgroup has finished the latest stage the
// inputs come from (x_after), so it overlaps any stage in between.
// sh.staged[sid] counts the stages this wave has staged.
__device__ void staging_wave(const ChainLaunch& L, Shared& sh, unsigned char* xl, int lane, int sid) {
    // Mark the other half of the copies empty for the next launch, which
    // writes and polls there (nothing in this launch reads it).  The halves
    // are multiples of 128 bytes.
    if (L.mirror_half_bytes) {
        const uint32_t other = L.mirror_half_bytes - sh.mirror_off;  // the half this launch does not use
        const __amdgpu_buffer_rsrc_t rm = make_rsrc(L.mirrors, 2u * L.mirror_half_bytes);
        const uint32_t e = kChainMirrorEmpty | (kChainMirrorEmpty << 16);
        const uint32_t n16 = L.mirror_half_bytes / 16u, step = (uint32_t)L.workers * kChainStagers * kWave;
        for (uint32_t i = ((uint32_t)blockIdx.x * kChainStagers + sid) * kWave + lane; i < n16; i += step)
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{e, e, e, e}, rm,
                                                   (int)(other + 16u * i), 0, kAuxDeviceCoherent);
    }
    for (int t = 0; t < L.num_stages; ++t) {
        // Buffer free: every compute wave here is past stage t - 2.  A stage
        // that reads earlier outputs also waits until this workgroup's own
        // part of the producing stage is done: by then the other workgroups'
        // parts are mostly done too, so the polls that follow are few
        // (polling from the start of the producing stage would load the
        // inputs over and over while the weights stream).
        const ChainStage& st = L.stages[t];
        const unsigned need = (unsigned)max(t - 1, st.x_internal ? st.x_after + 1 : 0);
        const bool ok = need == 0 || lds_wait(L, sh, [&] {
                            return __builtin_amdgcn_ballot_w64(
                                       lane < kChainComputeWaves &&
                                       lds_load(&sh.progress[lane < kChainComputeWaves ? lane : 0]) < need) == 0;
                        });
        if (lane == 0) timeline_mark(sh, t, 0, true);
        if (!ok || !stage_share(L, sh, t, xl + (size_t)(t & 1) * kChainXLdsBytes, lane, sid)) {
            set_error(L, sh, 8u);
            return;
        }
        if (lane == 0) __hip_atomic_store(&sh.staged[sid], (unsigned)t + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (lane == 0) timeline_mark(sh, t, 1, false);
    }
}

// --------------------------------------------------------------- compute wave
__device__ void compute_wave(const ChainLaunch& L, Shared& sh, const unsigned char* xl, int lane, int wi, int v,
                             int W) {
    // Report stages < upto done with (their LDS x is no longer read).
    auto report = [&](int upto) {
        if (lane == 0)
            __hip_atomic_store(&sh.progress[wi], (unsigned)upto, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    // Wait until stage s's x is staged.  On abort or time-out the wave goes on
    // without waiting (the outputs are then undefined; the error word says
    // so, bit 8 from a staging wave, bit 16 from a compute wave): leaving the
    // tile loop early instead makes the compiler's wait-count
    // analysis assume that the prefetched tiles were issued last, and wait for
    // all of them before every tile's math.
    auto staged = [&](int s) {
        return __builtin_amdgcn_ballot_w64(lane < kChainStagers &&
                                           lds_load(&sh.staged[lane < kChainStagers ? lane : 0]) <= (unsigned)s) == 0;
    };
    auto wait_x = [&](int s) {
        unsigned n = 0;
        bool r = staged(s), ab = lds_load(&sh.abort) != 0u;
        while (!r & !ab & (n <= L.spin_limit)) {
            __builtin_amdgcn_s_sleep(1);
            ++n;
            r = staged(s);
            ab = lds_load(&sh.abort) != 0u;
        }
        // A time-out is noted in LDS (an abort was recorded by whoever set
        // it); the workgroup writes the error bit at its end, so no global
        // store joins the tile loop.
        if (!r & !ab) __hip_atomic_store(&sh.timed_out, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };

    Work a = first_from(L, 0, v, W);
    report(a.s);  // no tiles in the first a.s stages; nothing pending
    int x_stage = -1;  // stage whose x this workgroup has staged and released

    if (a.s >= L.num_stages) return;

    // Three tiles in flight per wave, in three register sets used in turn:
    // while one tile is computed the next two load, and after the math the set
    // is refilled with the tile three ahead.  Past the wave's last tile the
    // refill is a dummy (an empty buffer range, which returns zeros without
    // touching memory), so every step issues the same loads and the
    // compiler's wait before a tile's math covers exactly that tile.  No wave
    // ever waits for its own stores: readers poll the output copies.
    TileRegs R0, R1, R2;
    const int S = L.num_stages;
    Work cur = a;
    Work nx1 = advance(L, cur, v, W);
    Work nx2 = nx1.s < S ? advance(L, nx1, v, W) : nx1;
    ChainGemv Gc = L.gemvs[cur.g];
    ChainGemv G1 = L.gemvs[nx1.s < S ? nx1.g : cur.g];
    ChainGemv G2 = L.gemvs[nx2.s < S ? nx2.g : cur.g];
    issue(Gc, cur, false, lane, R0);
    issue(G1, nx1.s < S ? nx1 : cur, nx1.s >= S, lane, R1);
    issue(G2, nx2.s < S ? nx2 : cur, nx2.s >= S, lane, R2);
    // Compute cur from Rc (the next two tiles are loading in the other sets);
    // refill Rc with the tile after them.  False once cur was the wave's last
    // tile.
    auto step = [&](TileRegs& Rc) -> bool {
        const bool has_n = nx1.s < S;
        const Work n3 = nx2.s < S ? advance(L, nx2, v, W) : nx2;
        const bool has_n3 = n3.s < S;
        const ChainGemv G3 = L.gemvs[has_n3 ? n3.g : cur.g];
        if (x_stage != cur.s) {
            wait_x(cur.s);
            x_stage = cur.s;
            if (lane == 0) timeline_mark(sh, cur.s, 2, true);
        }
        compute(Gc, cur, lane, Rc, xl + (size_t)(cur.s & 1) * kChainXLdsBytes + Gc.x_lds, sh.mirror_off,
                L.mirror_half_bytes);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        issue(G3, has_n3 ? n3 : cur, !has_n3, lane, Rc);
        if (nx1.s != cur.s) report(nx1.s);  // cur was this wave's last tile of its stage
        if (nx1.s != cur.s && lane == 0) timeline_mark(sh, cur.s, 3, false);
        if (!has_n) return false;
        cur = nx1;
        Gc = G1;
        nx1 = nx2;
        G1 = G2;
        nx2 = n3;
        G2 = G3;
        return true;
    };
    while (step(R0) && step(R1) && step(R2)) {
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

__global__ __launch_bounds__(kChainThreads) void chain_kernel(const ChainStage* __restrict__ stages,
                                                            const ChainGemv* __restrict__ gemvs, ChainLaunch L) {
    // The tables are read-only for the whole launch; as restrict kernel
    // arguments the compiler reads them with scalar loads, which do not
    // count in vmcnt (a vector load here would wait for every prefetch).
    L.stages = stages;
    L.gemvs = gemvs;
    __shared__ __attribute__((aligned(16))) unsigned char xl[2 * kChainXLdsBytes];
    __shared__ Shared sh;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    if (tid == 0) {
        for (int i = 0; i < kChainComputeWaves; ++i) sh.progress[i] = 0;
        for (int i = 0; i < kChainStagers; ++i) sh.staged[i] = 0;
        sh.abort = 0;
        sh.timed_out = 0;
        sh.base = L.counters[(size_t)blockIdx.x * kChainLineWords];
        sh.mirror_off = (sh.base & 1u) * L.mirror_half_bytes;
    }
#ifdef W4_CHAIN_TIMELINE
    for (int i = tid; i < kTimelineStages * 4; i += kChainThreads) sh.timeline[i] = (i & 1) ? 0u : ~0u;
#endif
    __syncthreads();
    if (wave >= 1 && wave <= kChainComputeWaves) {
        const int W = L.workers * kChainComputeWaves;
        // Position of this compute wave among the workgroup's in the stage
        // split.  Waves are placed on the 4 SIMDs in turn (wave w on SIMD
        // w % 4), so compute waves 1..8 sit two per SIMD; numbering them
        // 2 * SIMD + (first or second on it) makes the busy waves of a stage
        // with fewer tiles than waves (every second one, every fourth one)
        // land on different SIMDs instead of sharing two.  Any numbering is
        // correct; this one only spreads the work.
        const int l = 2 * (wave % 4) + (wave - 1) / 4;
        compute_wave(L, sh, xl, lane, wave - 1, uniform((int)blockIdx.x * kChainComputeWaves + l), W);
    } else {
        staging_wave(L, sh, xl, lane, wave == 0 ? 0 : wave - kChainComputeWaves);
    }
    // Every wave has left its loop (all waits are bounded): count the launch.
    // The next launch of the chain reads the counter only after this one ends.
    __syncthreads();
#ifdef W4_CHAIN_TIMELINE
    if (blockIdx.x < kTimelineWorkers)
        for (int i = tid; i < kTimelineStages * 4; i += kChainThreads)
            g_chain_timeline[blockIdx.x * kTimelineStages * 4 + i] = sh.timeline[i];
#endif
    if (tid == 0) {
        L.counters[(size_t)blockIdx.x * kChainLineWords] = sh.base + 1u;
        if (sh.timed_out) __hip_atomic_fetch_or(L.err, 16u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

hipError_t chain_occupancy(int* blocks_per_cu) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, chain_kernel, kChainThreads, 0);
}

hipError_t launch_chain(const ChainLaunch& l, hipStream_t stream) {
    chain_kernel<<<l.workers, kChainThreads, 0, stream>>>(l.stages, l.gemvs, l);
    return hipGetLastError();
}

}  // namespace w4

#ifdef W4_CHAIN_TIMELINE
// Timeline build only: copy the stamps of the last launch (unsigned
// [kTimelineWorkers][kTimelineStages][4], 100 MHz ticks) to host memory.
// Synchronises the device first.  Returns a hipError_t value.
extern "C" __attribute__((visibility("default"))) int w4_chain_timeline_read(void* host, size_t bytes) {
    hipError_t err = hipDeviceSynchronize();
    if (err == hipSuccess) err = hipMemcpyFromSymbol(host, HIP_SYMBOL(w4::g_chain_timeline), bytes);
    return (int)err;
}
#endif
