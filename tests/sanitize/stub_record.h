// What the last stubbed kernel launch was asked to do.
#pragma once
#include <cstdint>
struct StubRecord {
    int calls = 0;
    const char *what = "";
    int64_t a = 0, b = 0, c = 0;
    int n_split = 0;
};
extern StubRecord g_last;
