// Tables of the persistent decode-chain kernel, shared by the host planner
// (w4_api.hip) and the kernel (chain.hip).  They live in the caller's
// workspace, written once by w4_chain_create, beside the copies of
// the outputs that later GEMVs read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

// One INT4 GEMV of the chain.
struct ChainGemv {
    const void* qw;  // int32 [N][K/8]
    const void* s;   // fp16 [N][K/128]
    const void* z;   // fp16 [N][K/128]
    const void* x;   // bf16 [K]
    void* y;         // bf16 [N]
    int C;           // K / 32 chunks of 16 bytes per row
    int N;
    int sp;          // segments of 128 chunks per row: 1 (K <= 4096), 2 (K <= 8192) or 4 (K <= 16384)
    int tile0;       // first tile of this GEMV in its stage (tiles are kChainTileRows / sp rows)
    int x_lds;       // byte offset of this GEMV's staged x in its LDS buffer
    int x_internal;  // 1: x is the output of an earlier GEMV of the chain (read from xm)
    // Copies of outputs that later GEMVs read, in the first half of the
    // copies area (bf16 [N], padded to 64 values); a launch uses the half of
    // its parity.  ym: where this GEMV writes its own (null when no GEMV reads
    // its output); xm: its producer's, read instead of x (null when x comes
    // from outside the chain).
    uint16_t* ym;
    const uint16_t* xm;
    int xm_stage;  // stage index of xm's writer
    int x_slots;   // 64-chunk staging slots of x; 0 when an earlier GEMV of the stage has the same x
};

// GEMVs gemv0 .. gemv0 + ngemv - 1 form one stage: they run concurrently;
// every one of them starts after all earlier stages have written their outputs.
struct ChainStage {
    int gemv0;
    int ngemv;
    int tiles;       // total tiles of the stage's GEMVs
    int x_internal;  // 1: some input of the stage is an output of an earlier GEMV
    int x_after;     // latest stage whose outputs the stage reads (-1: none)
};

constexpr int kChainThreads = 768;  // 12 waves (3 per SIMD): kChainComputeWaves compute, the rest staging
constexpr int kChainComputeWaves = 8;
constexpr int kChainStagers = kChainThreads / 64 - kChainComputeWaves;  // staging waves
constexpr int kChainMaxWorkers = 1024;
constexpr int kChainTileRows = 4;     // slot-rows per compute-wave tile: 4 / sp rows of a GEMV
constexpr int kChainLineWords = 32;    // one 128-byte line per launch counter
constexpr int kChainMaxC = 512;        // K <= 16384
constexpr int kChainXLdsBytes = 65536; // staged x (pairs + chunk sums) of one stage; two buffers

// Staged x of one GEMV is zero-padded to the sp segments of 128 chunks its
// tiles read (128, 256 or 512 chunks), so the kernel never masks a chunk index.
__host__ __device__ inline int chain_x_chunks(int C) { return C <= 128 ? 128 : (C <= 256 ? 256 : 512); }
// Bytes of LDS one GEMV's staged x takes: 64 bytes of bf16 pairs and one
// FP32 sum per (padded) chunk.
__host__ __device__ inline int chain_x_lds_bytes(int C) { return 68 * chain_x_chunks(C); }

// Workspace layout: [error line][per-workgroup launch counter lines][stages]
// [gemvs][output copies: two halves of mirror_words bf16 values].
struct ChainLayout {
    size_t err, counters, stages, gemvs, mirrors, total;
};

inline ChainLayout chain_layout(int num_gemvs, int num_stages, size_t mirror_words) {
    const size_t line = kChainLineWords * 4;
    ChainLayout l;
    l.err = 0;
    l.counters = line;
    l.stages = l.counters + (size_t)kChainMaxWorkers * line;
    l.gemvs = l.stages + (size_t)num_stages * sizeof(ChainStage);
    l.gemvs = (l.gemvs + 63) & ~(size_t)63;
    l.mirrors = l.gemvs + (size_t)num_gemvs * sizeof(ChainGemv);
    l.mirrors = (l.mirrors + 255) & ~(size_t)255;
    l.total = l.mirrors + mirror_words * 2 * 2;
    return l;
}

struct ChainLaunch {
    const ChainStage* stages;
    const ChainGemv* gemvs;
    unsigned* err;
    unsigned* counters;  // one line per workgroup: launches it has run
    int num_stages;
    int workers;  // workgroups, one per compute unit
    unsigned spin_limit;
    uint16_t* mirrors;           // the output copies: two halves of mirror_half_bytes
    uint32_t mirror_half_bytes;  // 2 * mirror_words (a multiple of 128)
};

// A value of an output copy that is not written yet: a NaN pattern.  The
// halves are filled with it before use; a producer whose output has exactly
// these bits stores kChainMirrorNaN instead.
constexpr uint16_t kChainMirrorEmpty = 0xFFFFu;
constexpr uint16_t kChainMirrorNaN = 0x7FC0u;

hipError_t launch_chain(const ChainLaunch& l, hipStream_t stream);
hipError_t chain_occupancy(int* blocks_per_cu);

}  // namespace w4
