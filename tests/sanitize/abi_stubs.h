// What the host-only stand-ins of abi_stubs.cpp recorded.
#pragma once
#include "mxg_internal.h"

struct StubLog {
    int launches = 0;
    int copies = 0;
    const char* last = "";
    mxg::GemmProblem gemm{};
};
extern StubLog g_stub;
