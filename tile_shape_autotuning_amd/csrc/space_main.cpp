// Prints the kernel instantiation set: every configuration of the candidate
// space (split-K is a run-time value, so split_k = 1 only) that passes the
// shape-independent rules.  Used by the build to generate instantiation units.
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
            if (c.split_k != 1 || tg::check_static(dt, c, d) != tg::OK)
                continue;
            std::printf("%d %d %d %d %d %d %d %d\n", in_bf16, c.kind, c.bm, c.bn, c.bk, c.wgm, c.wgn, c.stages);
        }
    }
    return 0;
}
