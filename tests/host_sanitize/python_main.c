/* A Python interpreter whose executable carries the AddressSanitizer and
 * UndefinedBehaviorSanitizer runtimes, so that a library built with those
 * checks (its host code only) can be loaded by the ordinary Python tests. */
#include <Python.h>

int main(int argc, char** argv) { return Py_BytesMain(argc, argv); }
