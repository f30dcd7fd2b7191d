// One launch for a mixed step: the split-key decode pass and the chunked
// prefill tiles in a single grid.
//
// The pages' kernel covers whatever the scheduler packed into a step --
// prefill chunks, decode tokens, verify windows -- with one launch
// (vllm-metal v0.4.0 release post, "Replacing attention, reusing the rest").
// On MI355X the two halves cannot share a compute unit: a prefill workgroup
// holds 145 KiB of the 160 KiB LDS and two waves of ~230 VGPRs on every SIMD,
// and a decode wave needs ~250 VGPRs of its own.  So the single launch runs
// them in phases inside each workgroup: its first waves stream decode units
// (exactly the waves of the separate decode kernel, with their LDS carved out
// of the prefill ring), and the whole workgroup computes its prefill tile.
// Half the workgroups that carry both run their tile first and their decode
// waves after it, the rest the other way round, so that the decode streams are
// spread over the launch instead of all competing for HBM at its start while
// the matrix cores idle.  There is no grid-wide wait between the phases, and
// workgroups without a tile leave their compute unit to the tiles queued
// behind them.  Each decode wave and each tile does
// the same work, in the same order, as in the separate kernels, so the output
// is bitwise the same; the merge of cut decode segments stays a launch of its
// own after this one.
#pragma once

#include "decode.hpp"
#include "prefill.hpp"

namespace pkv {

struct StepParams {
    DecodeParams dp;
    PrefillParams pp;
    int decode_wgs;     // workgroups [0, decode_wgs) run decode waves ...
    int decode_per_wg;  // ... in their first decode_per_wg waves
    int prefill_wgs;    // workgroups [0, prefill_wgs) then run their prefill tile
    int tile_first;     // of every 4 workgroups of an XCD that carry both, this
                        // many run their tile first and their decode waves after
};

// Decode waves per workgroup and the workgroups that carry them, so that
// there are kDecodeWaves in all (decode_wgs is a multiple of the XCD count).
template <typename T>
constexpr int kStepWaves = kPrefillThreads<T> / kWave;

template <typename T, int D, bool LONG>
constexpr size_t step_lds_bytes() {
    return sizeof(PrefillLds<T, D, LONG>) > kStepWaves<T> * sizeof(DecodeLds<T, D>)
               ? sizeof(PrefillLds<T, D, LONG>)
               : kStepWaves<T> * sizeof(DecodeLds<T, D>);
}

template <typename T, int D, bool LONG>
__global__ void __launch_bounds__(kPrefillThreads<T>) step_kernel(StepParams sp) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[step_lds_bytes<T, D, LONG>()];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int b = (int)blockIdx.x;
    auto decode_part = [&]() {
        if (b < sp.decode_wgs && wave < sp.decode_per_wg) {
            // the decode wave numbers of XCD b % 8 stay one contiguous range, as
            // in the separate decode kernel (workgroups go to the XCDs in turn)
            const int w = (b % kXcds) * (kDecodeWaves / kXcds) + (b / kXcds) * sp.decode_per_wg + wave;
            decode_wave<T, D, false>(sp.dp, w, reinterpret_cast<DecodeLds<T, D>*>(lds)[wave]);
        }
    };
    // uniform over the workgroup
    if (b < sp.prefill_wgs && b < sp.decode_wgs && ((b / kXcds) & 3) < sp.tile_first) {
        prefill_tile<T, D, LONG>(sp.pp, b, *reinterpret_cast<PrefillLds<T, D, LONG>*>(lds));
        __syncthreads();  // the tile is done with the LDS
        decode_part();
        return;
    }
    decode_part();
    if (b >= sp.prefill_wgs) return;  // uniform over the workgroup
    __syncthreads();                  // the decode waves are done with the LDS
    prefill_tile<T, D, LONG>(sp.pp, b, *reinterpret_cast<PrefillLds<T, D, LONG>*>(lds));
}

}  // namespace pkv
