// Prints the kernel instantiation set: every configuration of the candidate
// space that passes the shape-independent rules, with split_k = 1 where
// split-K is a run-time value, and one kernel per K-group count for the
// sliced-K kind (its split_k is compiled in).  Fields: in_bf16 kind bm bn bk
// wgm wgn stages k_groups (0 where split_k is a run-time value).  Used by the
// build to generate instantiation units.
#include <cstdio>

#include "select.hpp"

// no kernel exists yet: the rules use their estimates only
bool tg::compiled_alloc(int, const tg_cfg&, tg::Alloc*) { return false; }

int main()
{
    const tg_device_desc d = tg::mi355x_desc();
    // fp32 operands: dtype TG_F32; bf16 operands: TG_BF16 (TG_BF16_F32OUT has the same space)
    const int dtypes[2] = {TG_F32, TG_BF16};
    for (int in_bf16 = 0; in_bf16 < 2; ++in_bf16) {
        const int dt = dtypes[in_bf16];
        for (const tg_cfg& c : tg::space(dt, d)) {
            const bool sliced = c.kind == TG_KIND_SLICEDK;
            if ((!sliced && c.split_k != 1) || tg::check_static(dt, c, d) != tg::OK)
                continue;
            std::printf("%d %d %d %d %d %d %d %d %d\n", in_bf16, c.kind, c.bm, c.bn, c.bk, c.wgm, c.wgn, c.stages,
                        sliced ? c.split_k : 0);
        }
    }
    return 0;
}
