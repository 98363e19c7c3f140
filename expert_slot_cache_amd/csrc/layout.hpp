// Byte layout of one expert as the library stores it (regions in order, each on a
// 256-byte boundary): f32/bf16: w13 [2I][H], w2 [H][I]; int4-g128: w13 codes
// [2I][H/8] u32, w2 codes [H][I/8] u32, s13 [2I][H/128] bf16, s2 [H][I/128] bf16
// ("Running 125B MoE on Two 32 GB Cards", section 1: an INT4 g128 expert is its codes
// plus bf16 scales).
#pragma once

#include <cstddef>
#include <cstdint>

#include "moe_pool.h"

namespace moe {

struct Layout {
    size_t off_w13 = 0, off_w2 = 0, off_s13 = 0, off_s2 = 0, total = 0;
};

inline size_t layout_round_up(size_t n) { return (n + 255) / 256 * 256; }

inline bool make_layout(int32_t wtype, int32_t H, int32_t I, Layout* L) {
    if (H <= 0 || I <= 0) return false;
    size_t w13, w2, s13 = 0, s2 = 0;
    if (wtype == MOE_W_F32) {
        if (H % 4 || I % 4) return false;
        w13 = (size_t)2 * I * H * 4;
        w2 = (size_t)H * I * 4;
    } else if (wtype == MOE_W_BF16) {
        if (H % 8 || I % 8) return false;
        w13 = (size_t)2 * I * H * 2;
        w2 = (size_t)H * I * 2;
    } else if (wtype == MOE_W_INT4_G128) {
        if (H % 128 || I % 128) return false;
        w13 = (size_t)I * H;           // 2I rows x H/2 bytes
        w2 = (size_t)H * I / 2;
        s13 = (size_t)2 * I * (H / 128) * 2;
        s2 = (size_t)H * (I / 128) * 2;
    } else {
        return false;
    }
    L->off_w13 = 0;
    L->off_w2 = layout_round_up(w13);
    size_t end = layout_round_up(L->off_w2 + w2);
    if (wtype == MOE_W_INT4_G128) {
        L->off_s13 = end;
        L->off_s2 = layout_round_up(L->off_s13 + s13);
        end = layout_round_up(L->off_s2 + s2);
    } else {
        L->off_s13 = L->off_s2 = 0;
    }
    L->total = end;
    return true;
}

}  // namespace moe
