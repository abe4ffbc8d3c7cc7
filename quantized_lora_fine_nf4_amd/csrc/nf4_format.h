// nf4_format.h -- constants of the NF4 format as the kernels embed them.
//
// The 16 levels are normal quantiles at evenly spaced probabilities, scaled so
// the outermost are -1 and +1, with an exact 0 ("QLoRA" paper summary page,
// ai360xpert.com, How It Works, NF4 item: 16 values with an equal share of
// normally distributed weights).  Reading taken where the page gives no
// formula: 7 negative and 8 positive quantiles, probabilities stepping evenly
// from 929/960 down to 1/2 on each side, divided by the quantile at 929/960,
// rounded to fp32.  The thresholds are the exact midpoints of neighbouring
// levels rounded toward minus infinity to fp32, so that "threshold < s" is
// exactly "s is nearer the upper level" (ties go to the lower code).
//
// Stored as fp32 bit patterns.
#pragma once
#include <stdint.h>

namespace nf4fmt {

constexpr int kBlock = 64;        // elements per absmax block
constexpr int kGroup = 256;       // absmax values per int8 double-quant group

constexpr uint32_t kLevelBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu,
    0xbe91a24bu, 0xbe3d353du, 0xbdba7869u, 0x00000000u,
    0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u,
};

constexpr uint32_t kThresholdBits[15] = {
    0xbf591cd9u, 0xbf1c5270u, 0xbeeb847du, 0xbeadea75u, 0xbe703ceau,
    0xbe0d38b9u, 0xbd3a7869u, 0x3d22fb01u, 0x3df6485fu, 0x3e5067dcu,
    0x3e9582d1u, 0x3ec753f5u, 0x3f006d01u, 0x3f248dacu, 0x3f5c89d8u,
};

}  // namespace nf4fmt
